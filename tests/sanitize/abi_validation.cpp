// Drives the host side of every C-ABI entry point (validation, workspace
// layout, parameter packing) under the address and undefined-behaviour
// sanitizers, with the kernel launchers replaced by counting stand-ins
// (launch_stubs.cpp).  Pointers are fake but aligned: nothing dereferences a
// tensor pointer on the host.  Prints "abi validation: N checks passed" or
// the first failing check and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "dn.h"

extern int g_launches;
extern int g_fail;

static int n_checks = 0;

#define EXPECT(call, want, launches_added)                                             \
  do {                                                                                  \
    const int before_ = g_launches;                                                     \
    const dn_status got_ = (call);                                                      \
    ++n_checks;                                                                         \
    if (got_ != (want) || g_launches - before_ != (launches_added)) {                  \
      fprintf(stderr, "line %d: %s -> %d (want %d), launches %d (want %d)\n", __LINE__, \
              #call, (int)got_, (int)(want), g_launches - before_, (launches_added));   \
      exit(1);                                                                          \
    }                                                                                   \
  } while (0)

static void *P(uintptr_t x) { return reinterpret_cast<void *>(x << 8); }  // aligned fake address
static float *F(uintptr_t x) { return reinterpret_cast<float *>(x << 8); }

static dn_shape shape(int B, int T, int H, int Dk, int Dv, int N, int chunk, int dt) {
  dn_shape s;
  s.B = B; s.T = T; s.H = H; s.Dk = Dk; s.Dv = Dv; s.n_seqs = N; s.chunk = chunk; s.dtype = dt;
  return s;
}

static dn_status fwd(const dn_shape *s, const int32_t *cu, void *o = P(20), void *ws = nullptr, size_t wsb = 0) {
  return dn_chunk_fwd(s, P(1), P(2), P(3), F(4), F(5), F(6), cu, o, F(21), ws, wsb, nullptr);
}

static dn_status bwd(const dn_shape *s, const int32_t *cu, size_t ws, const float *g = F(5), float *dg = F(34),
                     const void *q = P(1)) {
  return dn_chunk_bwd(s, q, P(2), P(3), F(4), g, F(6), cu, P(7), F(8), F(30), F(31), F(32), F(33), dg, F(35),
                      P(40), ws, nullptr);
}

int main() {
  const int32_t *cu = reinterpret_cast<const int32_t *>(P(9));
  // ---- status strings
  for (int i = 0; i <= 5; ++i)
    if (!dn_status_str((dn_status)i)) return 1;

  // ---- forward
  dn_shape s = shape(2, 300, 4, 128, 256, 2, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_OK, 1);
  EXPECT(fwd(nullptr, nullptr), DN_EINVAL, 0);
  s.chunk = 32;
  EXPECT(fwd(&s, nullptr), DN_OK, 1);
  s.chunk = 128;
  EXPECT(fwd(&s, nullptr), DN_EUNSUPPORTED, 0);
  s = shape(2, 300, 4, 128, 256, 2, 32, DN_F32);
  EXPECT(fwd(&s, nullptr), DN_EUNSUPPORTED, 0);  // 32-token chunks are bf16 only
  s = shape(2, 300, 4, 96, 256, 2, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EUNSUPPORTED, 0);
  s = shape(2, 300, 4, 128, 1088, 2, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EUNSUPPORTED, 0);
  s = shape(2, 300, 4, 128, 96, 2, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EUNSUPPORTED, 0);
  s = shape(2, 300, 4, 128, 128, 2, 64, DN_F32);
  EXPECT(fwd(&s, nullptr), DN_EUNSUPPORTED, 0);  // fp32 runs d_k = 64 only
  s = shape(2, 300, 4, 64, 128, 2, 64, DN_F32);
  EXPECT(fwd(&s, nullptr), DN_OK, 1);
  s = shape(2, -1, 4, 128, 128, 2, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EINVAL, 0);
  s = shape(0, 10, 4, 128, 128, 0, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EINVAL, 0);
  s = shape(2, 10, 4, 128, 128, 3, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EINVAL, 0);  // n_seqs != B without offsets
  s = shape(2, 10, 4, 128, 128, 3, 64, DN_BF16);
  EXPECT(fwd(&s, cu), DN_EINVAL, 0);       // offsets need B == 1
  s = shape(1, 10, 4, 128, 128, 3, 64, DN_BF16);
  // packed input: the workspace holds the longest-first sequence order (3 entries, one 256-byte block)
  if (dn_chunk_fwd_workspace(&s) != 256) return 1;
  EXPECT(fwd(&s, cu), DN_ENOWS, 0);
  EXPECT(fwd(&s, cu, P(20), P(41), 255), DN_ENOWS, 0);
  EXPECT(fwd(&s, cu, P(20), reinterpret_cast<char *>(P(41)) + 4, 256), DN_ENOWS, 0);  // misaligned
  EXPECT(fwd(&s, cu, P(20), P(41), 256), DN_OK, 2);  // the order, then the forward kernel
  s.chunk = 32;
  EXPECT(fwd(&s, cu, P(20), P(41), 256), DN_OK, 2);
  s = shape(2, 10, 4, 128, 128, 2, 64, DN_BF16);
  if (dn_chunk_fwd_workspace(&s) != 0) return 1;  // fixed-length input needs none
  s = shape(1, 10, 4, 128, 128, 70000, 64, DN_BF16);
  if (dn_chunk_fwd_workspace(&s) != 0) return 1;  // packs above 65536 sequences keep their own order
  EXPECT(fwd(&s, cu), DN_OK, 1);
  s = shape(1, 10, 4, 128, 128, 1, 64, 7);
  EXPECT(fwd(&s, nullptr), DN_EINVAL, 0);
  s = shape(1, 10, 4, 128, 128, 1, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr, nullptr), DN_EINVAL, 0);  // no output
  EXPECT(dn_chunk_fwd(&s, reinterpret_cast<char *>(P(1)) + 4, P(2), P(3), F(4), F(5), F(6), nullptr, P(20), F(21),
                      nullptr, 0, nullptr),
         DN_EINVAL, 0);  // misaligned q
  s = shape(1, 0, 4, 128, 128, 1, 64, DN_BF16);
  EXPECT(dn_chunk_fwd(&s, nullptr, nullptr, nullptr, nullptr, nullptr, F(6), nullptr, nullptr, F(21), nullptr, 0,
                      nullptr),
         DN_OK, 1);  // T = 0: only the state is passed through
  // limits: the byte span of one chunk of fp32 rows must fit 32-bit offsets
  s = shape(1, 64, 1 << 20, 128, 1024, 1, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EUNSUPPORTED, 0);
  s = shape(1 << 20, 1 << 20, 1 << 12, 128, 1024, 1 << 20, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EUNSUPPORTED, 0);
  s = shape(INT32_MAX, INT32_MAX, 1, 64, 64, INT32_MAX, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EUNSUPPORTED, 0);
  s = shape(1, INT32_MAX, 1, 64, 64, 1, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_OK, 1);

  // ---- backward and its workspace
  s = shape(2, 300, 4, 128, 256, 2, 64, DN_BF16);
  const size_t ws = dn_chunk_bwd_workspace(&s);
  // chunk-start states and their gradients, bf16, per (chunk, head)
  if (ws != 2 * (size_t)(2 * 5) * 4 * 128 * 256 * 2) {
    fprintf(stderr, "workspace %zu\n", ws);
    return 1;
  }
  EXPECT(bwd(&s, nullptr, ws), DN_OK, 2);      // recompute, then scan + chunk kernel
  EXPECT(bwd(&s, nullptr, ws - 1), DN_ENOWS, 0);
  EXPECT(bwd(&s, nullptr, ws, nullptr), DN_EINVAL, 0);           // dg without g
  EXPECT(bwd(&s, nullptr, ws, F(5), nullptr), DN_EINVAL, 0);     // g without dg
  EXPECT(bwd(&s, nullptr, ws, nullptr, nullptr), DN_OK, 2);      // ungated
  EXPECT(bwd(&s, nullptr, ws, F(5), F(34), nullptr), DN_EINVAL, 0);
  s.dtype = DN_F32;
  EXPECT(bwd(&s, nullptr, ws), DN_EUNSUPPORTED, 0);
  s = shape(1, 300, 4, 128, 256, 5, 64, DN_BF16);
  const size_t wsv = dn_chunk_bwd_workspace(&s);
  EXPECT(bwd(&s, cu, wsv), DN_OK, 4);          // chunk table, sequence order, recompute, backward
  EXPECT(bwd(&s, cu, wsv - 1), DN_ENOWS, 0);
  s = shape(1, 0, 4, 128, 256, 3, 64, DN_BF16);
  EXPECT(dn_chunk_bwd(&s, nullptr, nullptr, nullptr, nullptr, F(5), F(6), cu, nullptr, F(8), nullptr, nullptr,
                      nullptr, nullptr, F(34), F(35), nullptr, dn_chunk_bwd_workspace(&s), nullptr),
         DN_ENOWS, 0);  // packed, all empty: the workspace still holds the chunk table
  EXPECT(dn_chunk_bwd(&s, nullptr, nullptr, nullptr, nullptr, F(5), F(6), cu, nullptr, F(8), nullptr, nullptr,
                      nullptr, nullptr, F(34), F(35), P(40), dn_chunk_bwd_workspace(&s), nullptr),
         DN_OK, 4);
  if (dn_chunk_bwd_workspace(nullptr) != 0) return 1;
  s = shape(1, INT32_MAX, 1 << 12, 128, 1024, 1, 64, DN_BF16);
  EXPECT(bwd(&s, nullptr, (size_t)-1), DN_EUNSUPPORTED, 0);  // too many (chunk, head) pairs

  // ---- the training pair
  s = shape(2, 300, 4, 128, 256, 2, 64, DN_BF16);
  EXPECT(dn_chunk_fwd_save(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(20), F(21), P(40), ws, nullptr),
         DN_OK, 1);
  EXPECT(dn_chunk_fwd_save(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(20), F(21), P(40), ws - 256,
                           nullptr),
         DN_ENOWS, 0);
  EXPECT(dn_chunk_bwd_saved(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(7), F(8), F(30), F(31), F(32),
                            F(33), F(34), F(35), P(40), ws, nullptr, nullptr),
         DN_OK, 1);
  EXPECT(dn_chunk_bwd_prologue(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(7), F(8), P(11), P(12), F(13),
                               0.1f, F(30), F(31), F(32), F(33), F(34), F(35), P(40), ws, nullptr, nullptr),
         DN_OK, 1);
  EXPECT(dn_chunk_bwd_prologue(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(7), F(8), P(11), P(12), nullptr,
                               0.1f, F(30), F(31), F(32), F(33), F(34), F(35), P(40), ws, nullptr, nullptr),
         DN_EINVAL, 0);  // gate without its raw input
  EXPECT(dn_chunk_bwd_longhorn(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(7), F(8), F(14), F(30), F(31),
                               F(32), F(33), F(34), F(35), P(40), ws, nullptr, nullptr),
         DN_OK, 1);
  EXPECT(dn_chunk_bwd_longhorn(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(7), F(8), nullptr, F(30), F(31),
                               F(32), F(33), F(34), F(35), P(40), ws, nullptr, nullptr),
         DN_EINVAL, 0);

  // ---- 32-token chunks: the training pair and the backward pass (ceil(300 / 32) = 10 chunks per sequence)
  s = shape(2, 300, 4, 128, 256, 2, 32, DN_BF16);
  const size_t ws32 = dn_chunk_bwd_workspace(&s);
  if (ws32 != 2 * (size_t)(2 * 10) * 4 * 128 * 256 * 2) {
    fprintf(stderr, "32-token workspace %zu\n", ws32);
    return 1;
  }
  EXPECT(bwd(&s, nullptr, ws32), DN_OK, 2);
  EXPECT(bwd(&s, nullptr, ws), DN_ENOWS, 0);  // sized for 64-token chunks
  EXPECT(dn_chunk_fwd_save(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(20), F(21), P(40), ws32, nullptr),
         DN_OK, 1);
  EXPECT(dn_chunk_bwd_saved(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(7), F(8), F(30), F(31), F(32),
                            F(33), F(34), F(35), P(40), ws32, nullptr, nullptr),
         DN_OK, 1);
  EXPECT(dn_chunk_bwd_prologue(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(7), F(8), P(11), P(12), F(13),
                               0.1f, F(30), F(31), F(32), F(33), F(34), F(35), P(40), ws32, nullptr, nullptr),
         DN_EUNSUPPORTED, 0);  // the folded variants take 64-token chunks
  EXPECT(dn_chunk_bwd_longhorn(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(7), F(8), F(14), F(30), F(31),
                               F(32), F(33), F(34), F(35), P(40), ws32, nullptr, nullptr),
         DN_EUNSUPPORTED, 0);
  s = shape(1, 300, 4, 128, 256, 5, 32, DN_BF16);
  EXPECT(bwd(&s, cu, dn_chunk_bwd_workspace(&s)), DN_OK, 4);  // chunk table, order, recompute, backward

  // ---- decode step
  EXPECT(dn_recurrent_step(256, 32, 128, 128, DN_BF16, P(1), P(2), P(3), F(4), F(5), F(6), P(7), nullptr), DN_OK,
         1);
  EXPECT(dn_recurrent_step(256, 32, 128, 128, DN_BF16, P(1), P(2), P(3), F(4), F(5), nullptr, P(7), nullptr),
         DN_EINVAL, 0);
  EXPECT(dn_recurrent_step(256, 32, 100, 128, DN_BF16, P(1), P(2), P(3), F(4), F(5), F(6), P(7), nullptr),
         DN_EUNSUPPORTED, 0);
  EXPECT(dn_recurrent_step(0, 32, 128, 128, DN_BF16, P(1), P(2), P(3), F(4), F(5), F(6), P(7), nullptr), DN_EINVAL,
         0);

  // ---- row passes around the recurrence
  EXPECT(dn_longhorn_eps(2, 100, 4, 128, DN_BF16, P(1), F(2), F(3), nullptr), DN_OK, 1);
  EXPECT(dn_longhorn_eps(2, 0, 4, 128, DN_BF16, nullptr, nullptr, nullptr, nullptr), DN_OK, 0);
  EXPECT(dn_longhorn_eps(INT32_MAX, INT32_MAX, 4, 128, DN_BF16, P(1), F(2), F(3), nullptr), DN_EUNSUPPORTED, 0);
  EXPECT(dn_longhorn_eps_bwd(2, 100, 4, 128, DN_BF16, P(1), F(2), F(3), F(4), F(5), nullptr), DN_OK, 1);
  EXPECT(dn_longhorn_eps_bwd(2, 100, 4, 128, DN_BF16, P(1), F(2), F(3), nullptr, F(5), nullptr), DN_EINVAL, 0);
  EXPECT(dn_prologue(2, 100, 4, 128, DN_BF16, P(1), P(2), F(3), F(4), 0.1f, P(5), P(6), F(7), F(8), nullptr), DN_OK,
         1);
  EXPECT(dn_prologue(2, 100, 4, 128, DN_BF16, P(1), P(2), F(3), nullptr, 0.1f, P(5), P(6), F(7), F(8), nullptr),
         DN_EINVAL, 0);
  EXPECT(dn_prologue_bwd(2, 100, 4, 128, DN_BF16, P(1), P(2), F(3), F(4), 0.1f, F(5), F(6), F(7), F(8), F(9),
                         F(10), F(11), F(12), nullptr),
         DN_OK, 1);
  EXPECT(dn_short_conv(2, 100, 4, 128, 4, 2, DN_BF16, P(1), F(2), nullptr, P(3), nullptr), DN_OK, 1);
  EXPECT(dn_short_conv(2, 100, 4, 128, 5, 2, DN_BF16, P(1), F(2), nullptr, P(3), nullptr), DN_EUNSUPPORTED, 0);
  EXPECT(dn_short_conv(2, 100, 4, 128, 4, 2, DN_BF16, P(1), F(2), cu, P(3), nullptr), DN_EINVAL, 0);
  EXPECT(dn_short_conv_bwd(1, 100, 4, 128, 4, 3, DN_BF16, P(1), F(2), cu, F(3), F(4), F(5), nullptr), DN_OK, 1);
  EXPECT(dn_short_conv_bwd(1, 100, 4, 128, 4, 3, DN_BF16, P(1), F(2), cu, F(3), F(4), nullptr, nullptr), DN_EINVAL,
         0);
  EXPECT(dn_short_conv_l2(2, 100, 4, 96, 4, 2, DN_BF16, P(1), F(2), nullptr, P(3), nullptr), DN_EUNSUPPORTED, 0);
  EXPECT(dn_short_conv_l2(2, 100, 4, 128, 4, 2, DN_BF16, P(1), F(2), nullptr, P(3), nullptr), DN_OK, 1);
  EXPECT(dn_short_conv_l2_bwd(2, 100, 4, 64, 2, 2, DN_F32, P(1), F(2), nullptr, F(3), F(4), F(5), nullptr), DN_OK,
         1);
  EXPECT(dn_short_conv(1, INT32_MAX, 65535, 1024, 4, 1, DN_BF16, P(1), F(2), nullptr, P(3), nullptr),
         DN_EUNSUPPORTED, 0);

  // ---- a failed launch is reported as DN_EHIP, and nothing after it is launched
  g_fail = 1;
  s = shape(2, 300, 4, 128, 256, 2, 64, DN_BF16);
  EXPECT(fwd(&s, nullptr), DN_EHIP, 1);
  EXPECT(bwd(&s, nullptr, ws), DN_EHIP, 1);  // the recompute fails; the backward kernels are not launched
  EXPECT(dn_chunk_fwd_save(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(20), F(21), P(40), ws, nullptr),
         DN_EHIP, 1);
  EXPECT(dn_chunk_bwd_saved(&s, P(1), P(2), P(3), F(4), F(5), F(6), nullptr, P(7), F(8), F(30), F(31), F(32),
                            F(33), F(34), F(35), P(40), ws, nullptr, nullptr),
         DN_EHIP, 1);
  s = shape(1, 300, 4, 128, 256, 5, 64, DN_BF16);
  EXPECT(bwd(&s, cu, wsv), DN_EHIP, 1);  // the chunk table fails first
  s = shape(1, 10, 4, 128, 128, 3, 64, DN_BF16);
  EXPECT(fwd(&s, cu, P(20), P(41), 256), DN_EHIP, 1);  // the order fails; the forward is not launched
  EXPECT(dn_recurrent_step(256, 32, 128, 128, DN_BF16, P(1), P(2), P(3), F(4), F(5), F(6), P(7), nullptr), DN_EHIP,
         1);
  EXPECT(dn_short_conv(2, 100, 4, 128, 4, 2, DN_BF16, P(1), F(2), nullptr, P(3), nullptr), DN_EHIP, 1);
  EXPECT(dn_prologue(2, 100, 4, 128, DN_BF16, P(1), P(2), F(3), F(4), 0.1f, P(5), P(6), F(7), F(8), nullptr), DN_EHIP,
         1);
  g_fail = 0;

  printf("abi validation: %d checks passed\n", n_checks);
  return 0;
}
