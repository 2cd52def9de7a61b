/*
 * Host-side sweep of the C ABI: every size query and every rejection path
 * over a deterministic set of configurations, including negative, zero and
 * near-INT32_MAX fields.  Built together with the library's host code under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_abi_sanitized.py),
 * so an overflow or out-of-bounds access in the host checks aborts the run.
 * No call here reaches a HIP launch: every launching entry point gets a NULL
 * for a pointer it requires, or a configuration it rejects.
 * Prints "ok <configs> <accepted>" and exits 0 when every status is known.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static const int32_t kVals[] = {-2147483647 - 1, -1, 0, 1, 2, 3, 7, 8, 16, 32, 63, 64, 100, 128,
                                192, 256, 1024, 1025, 4096, 7168, 65536, 1 << 20, 1 << 30,
                                2147483647};
#define NVALS ((int)(sizeof(kVals) / sizeof(kVals[0])))

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64(void) { /* splitmix64 */
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
static int32_t pick(void) {
  /* half the draws from the interesting values, half small positive */
  const uint64_t r = next_u64();
  if (r & 1) return kVals[(r >> 1) % NVALS];
  return (int32_t)((r >> 8) % 300);
}

static int known(int s) {
  return s == MOE_OK || s == MOE_EINVAL || s == MOE_EUNSUPPORTED || s == MOE_ESCRATCH;
}

static int fails = 0;
static void expect(int cond, const char* what, const moe_config* c) {
  if (!cond) {
    ++fails;
    if (fails < 10 && !c) fprintf(stderr, "FAIL %s\n", what);
    if (fails < 10 && c)
      fprintf(stderr, "FAIL %s: T=%d d=%d E=%d k=%d f=%d g=%d/%d p=%d r=%d ep=%d dt=%d\n", what,
              c->T, c->d, c->E, c->k, c->f, c->n_group, c->topk_group, c->presel, c->renorm,
              c->ep_ranks, c->dtype);
  }
}

int main(void) {
  char fake_mem[64];
  void* fake = fake_mem; /* never dereferenced: every call below is rejected */
  long accepted = 0, n = 0;
  for (int s = -10; s <= 10; ++s) expect(moe_strerror(s) != NULL, "strerror", NULL);
  expect(moe_noalloc_scratch_bytes() > 0, "noalloc bytes", NULL);
  expect(moe_validate(NULL) == MOE_EINVAL, "validate(NULL)", NULL);

  for (int it = 0; it < 200000; ++it) {
    moe_config c;
    c.T = pick(); c.d = pick(); c.E = pick(); c.k = pick(); c.f = pick();
    c.n_group = pick(); c.topk_group = pick(); c.presel = pick();
    c.renorm = (int32_t)(next_u64() % 3) - (it % 7 == 0);
    c.ep_ranks = pick();
    c.dtype = (int32_t)(next_u64() % 3);
    if (it % 4 == 0) { /* mostly-valid shapes reach the size arithmetic */
      c.n_group = 1; c.topk_group = 1; c.presel = 0; c.renorm = 1; c.ep_ranks = 1;
      c.d = 64 * (1 + (int32_t)(next_u64() % 200));
      c.f = 64 * (1 + (int32_t)(next_u64() % 200));
      c.E = 1 + (int32_t)(next_u64() % 300);
      c.k = 1 + (int32_t)(next_u64() % 16);
    }
    ++n;
    const int v = moe_validate(&c);
    expect(known(v), "validate status", &c);
    if (v == MOE_OK) ++accepted;
    for (int entry = -1; entry <= 9; ++entry) {
      size_t b = 12345;
      const int s = moe_workspace_bytes(&c, entry, &b);
      expect(known(s), "workspace status", &c);
      expect(moe_workspace_bytes(&c, entry, NULL) == MOE_EINVAL, "workspace(NULL)", &c);
    }
    size_t g = 0, dn = 0;
    expect(known(moe_packed_weight_bytes(&c, &g, &dn)), "packed bytes", &c);
    expect(known(moe_packed_weight_bytes_backward(&c, &g, &dn)), "packed bytes bwd", &c);
    expect(known(moe_fp8_weight_bytes(&c, &g)), "fp8 bytes", &c);

    /* launching entry points with a required pointer missing: rejected
       (an empty batch, T = 0, may pass NULL for its zero-size arrays) */
    if (c.T == 0) continue;
    expect(moe_route(&c, fake, fake, NULL, fake, NULL, fake, NULL, 0, NULL) != MOE_OK,
           "route rejects", &c);
    expect(moe_permute(&c, NULL, NULL, fake, fake, fake, fake, NULL, NULL, 0, NULL) != MOE_OK,
           "permute rejects", &c);
    expect(moe_permute_noalloc(&c, NULL, NULL, fake, fake, fake, fake, NULL, NULL) != MOE_OK,
           "permute_noalloc rejects", &c);
    expect(moe_ffn_gate_up(&c, fake, NULL, fake, fake, fake, NULL) != MOE_OK, "gate_up rejects",
           &c);
    expect(moe_ffn_down(&c, fake, NULL, fake, fake, NULL) != MOE_OK, "down rejects", &c);
    expect(moe_combine(&c, fake, NULL, fake, fake, NULL) != MOE_OK, "combine rejects", &c);
    expect(moe_quantize_fp8(&c, fake, NULL, fake, NULL) != MOE_OK, "quantize rejects", &c);
    expect(moe_dequantize_fp8(&c, fake, NULL, fake, fake, NULL) != MOE_OK, "dequantize rejects",
           &c);
    expect(moe_ffn_gate_up_packed_gather(&c, fake, NULL, fake, fake, fake, NULL) != MOE_OK,
           "gather rejects", &c);
    expect(moe_ffn_gate_up_fp8_gather(&c, fake, fake, NULL, fake, fake, fake, NULL) != MOE_OK,
           "fp8 gather rejects", &c);
    expect(moe_pack_weights_fp8(&c, fake, NULL, fake, NULL) != MOE_OK, "fp8 pack rejects", &c);
    expect(moe_combine_backward(&c, fake, fake, NULL, fake, fake, fake, NULL) != MOE_OK,
           "combine bwd rejects", &c);
  }
  expect(moe_workspace_bytes(NULL, MOE_ENTRY_LAYER, NULL) == MOE_EINVAL, "ws(NULL)", NULL);
  if (fails) return 1;
  printf("ok %ld %ld\n", n, accepted);
  return 0;
}
