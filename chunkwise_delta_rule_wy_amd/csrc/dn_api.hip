// C ABI of the library: argument validation, workspace sizing and launches.
// Every entry point validates on the host and enqueues nothing on error; it
// never allocates, frees or synchronises.
#include "dn.h"
#include "dn_entry.h"
#include "dn_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int dtype) { return dtype == DN_BF16 ? 2 : 4; }

// chunk32: the pass also takes 32-token chunks (bf16 inputs)
dn_status check_shape(const dn_shape *s, const int32_t *cu, bool chunk32 = false) {
  if (!s) return DN_EINVAL;
  if (s->B <= 0 || s->T < 0 || s->H <= 0 || s->Dk <= 0 || s->Dv <= 0 || s->n_seqs <= 0)
    return DN_EINVAL;
  if (s->dtype != DN_F32 && s->dtype != DN_BF16) return DN_EINVAL;
  if (cu) {
    if (s->B != 1) return DN_EINVAL;
  } else if (s->n_seqs != s->B) {
    return DN_EINVAL;
  }
  if (s->chunk != 64 && !(chunk32 && s->chunk == 32 && s->dtype == DN_BF16)) return DN_EUNSUPPORTED;
  if (s->Dk != 64 && s->Dk != 128) return DN_EUNSUPPORTED;
  if (s->Dv % 64 != 0 || s->Dv > 1024) return DN_EUNSUPPORTED;
  if (s->dtype == DN_F32 && s->Dk != 64) return DN_EUNSUPPORTED;
  // element offsets are computed in 64-bit, but grid and per-sequence counts are int
  if ((int64_t)s->n_seqs * s->H * (s->Dv / 64) > (int64_t)1 << 30) return DN_EUNSUPPORTED;
  // the kernels address the rows of one chunk (64 tokens of one head, fp32 at
  // most) with 32-bit offsets from the chunk's first row
  if ((int64_t)64 * s->H * (s->Dk > s->Dv ? s->Dk : s->Dv) * 4 > INT32_MAX) return DN_EUNSUPPORTED;
  return DN_OK;
}

// Chunk length of a shape that passed check_shape (64 or 32).
int chunk_len(const dn_shape *s) { return s->chunk == 32 ? 32 : 64; }

// Upper bound on the number of chunks over all sequences.
int64_t max_chunks(const dn_shape *s, bool varlen) {
  const int C = chunk_len(s);
  if (!varlen) return (int64_t)s->B * (((int64_t)s->T + C - 1) / C);
  // sum_n ceil(L_n / C) <= floor(T / C) + n_seqs
  return (int64_t)s->T / C + s->n_seqs;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t states, dstates, table, total;
};

// Entries of the longest-first sequence order (packed input of at most
// MAX_ORDERED_SEQS sequences; larger packs keep their own order).
size_t order_len(const dn_shape *s, bool varlen) {
  return varlen && s->n_seqs <= dn::MAX_ORDERED_SEQS ? (size_t)s->n_seqs : 0;
}

// Backward workspace: bf16 chunk states and state gradients, then for packed
// input the chunk table (chunk_base [N + 1], chunk_seq [chunks]) and the
// sequence order [N].
BwdLayout bwd_layout(const dn_shape *s, bool varlen) {
  BwdLayout L;
  const size_t nch = (size_t)max_chunks(s, varlen);
  const size_t per = (size_t)s->H * s->Dk * s->Dv * 2;  // bf16 states
  L.states = 0;
  L.dstates = align256(nch * per);
  L.table = L.dstates + align256(nch * per);
  L.total = L.table +
            (varlen ? align256(sizeof(int32_t) * ((size_t)s->n_seqs + 1 + nch + order_len(s, varlen))) : 0);
  return L;
}

// Forward workspace: the sequence order of packed input (nothing otherwise).
size_t fwd_ws_bytes(const dn_shape *s, bool varlen) { return align256(sizeof(int32_t) * order_len(s, varlen)); }

dn_status from_hip(hipError_t e) { return e == hipSuccess ? DN_OK : DN_EHIP; }

dn::FwdParams fwd_params(const dn_shape *s, const void *q, const void *k, const void *v,
                         const float *beta, const float *g, const float *h0, const int32_t *cu) {
  dn::FwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.g = g;
  p.h0 = h0;
  p.cu = cu;
  p.B = s->B;
  p.T = s->T;
  p.H = s->H;
  p.DV = s->Dv;
  p.N = s->n_seqs;
  p.NC = (int)(((int64_t)s->T + chunk_len(s) - 1) / chunk_len(s));
  p.ntiles = s->Dv / 64;
  p.xcd_map = ((s->n_seqs * s->H) % 8) == 0;
  return p;
}

// Checks shared by the passes that use the backward workspace (bf16 only).
dn_status check_train(const dn_shape *s, const int32_t *cu, const void *q, const void *k, const void *v,
                      const float *beta) {
  dn_status st = check_shape(s, cu, true);
  if (st != DN_OK) return st;
  if (s->dtype != DN_BF16) return DN_EUNSUPPORTED;  // the backward kernels are bf16
  if (s->T > 0) {
    if (!q || !k || !v || !beta) return DN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return DN_EINVAL;
  }
  return DN_OK;
}

// Pieces of the backward workspace; builds the packed-sequence chunk table
// (varlen) on `stream`.
struct TrainWs {
  bf16 *states, *dstates;
  int32_t *chunk_base, *chunk_seq, *order;
  int64_t nchunks;
};

dn_status train_ws(const dn_shape *s, const int32_t *cu, void *workspace, size_t workspace_bytes,
                   hipStream_t stream, TrainWs &w) {
  const bool varlen = cu != nullptr;
  w.nchunks = max_chunks(s, varlen);
  // the chunk-parallel kernel launches one workgroup per (chunk, head)
  if (w.nchunks * s->H >= (int64_t)INT32_MAX) return DN_EUNSUPPORTED;
  // the workspace query cannot see cu_seqlens, so it sizes for the varlen bound
  const BwdLayout L = bwd_layout(s, varlen || s->B == 1);
  // a shape that needs no workspace (no chunk at all) accepts a null one
  if (workspace_bytes < L.total || (L.total > 0 && (!workspace || !aligned16(workspace)))) return DN_ENOWS;
  char *ws = static_cast<char *>(workspace);
  w.chunk_base = w.chunk_seq = w.order = nullptr;
  if (varlen) {
    w.chunk_base = reinterpret_cast<int32_t *>(ws + L.table);
    w.chunk_seq = w.chunk_base + s->n_seqs + 1;
    hipError_t e = dn::launch_chunk_table(cu, s->n_seqs, w.chunk_base, w.chunk_seq, (int)w.nchunks, chunk_len(s),
                                          stream);
    if (e != hipSuccess) return DN_EHIP;
    if (order_len(s, true) > 0) {
      w.order = w.chunk_seq + w.nchunks;
      if (dn::launch_seq_order(cu, s->n_seqs, w.order, stream) != hipSuccess) return DN_EHIP;
    }
  }
  w.states = reinterpret_cast<bf16 *>(ws + L.states);
  w.dstates = reinterpret_cast<bf16 *>(ws + L.dstates);
  return DN_OK;
}

}  // namespace

namespace dn {

dn_status bwd_check(const dn_shape *s, const void *q, const void *k, const void *v, const float *beta,
                    const float *g, const int32_t *cu_seqlens, const void *dO, const float *dq, const float *dk,
                    const float *dv, const float *dbeta, const float *dg) {
  dn_status st = check_train(s, cu_seqlens, q, k, v, beta);
  if (st != DN_OK) return st;
  if ((g == nullptr) != (dg == nullptr)) return DN_EINVAL;
  if (s->T > 0) {
    if (!dO || !dq || !dk || !dv || !dbeta) return DN_EINVAL;
    if (!aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return DN_EINVAL;
  }
  return DN_OK;
}

}  // namespace dn

namespace {

// Raw inputs of the input prologue, or the Longhorn step size's beta, when
// their backward is folded into the chunk-gradient kernel.
struct ProIn {
  const void *q_in = nullptr, *k_in = nullptr;
  const float *x_in = nullptr;
  float gate_scale = 0.f;
  const float *beta_raw = nullptr;
};

// The backward pass.  With `recompute` false it reads the chunk-start states
// that the saving forward pass left in the workspace instead of recomputing
// them; with pro.q_in set the gradient outputs are those of the prologue's
// raw inputs.
dn_status bwd_run(const dn_shape *s, const void *q, const void *k, const void *v, const float *beta,
                  const float *g, const float *h0, const int32_t *cu_seqlens, const void *dO,
                  const float *dhT, float *dq, float *dk, float *dv, float *dbeta, float *dg, float *dh0,
                  void *workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t *events,
                  bool recompute, const ProIn &pro = ProIn()) {
  dn_status st = dn::bwd_check(s, q, k, v, beta, g, cu_seqlens, dO, dq, dk, dv, dbeta, dg);
  if (st != DN_OK) return st;
  TrainWs w;
  st = train_ws(s, cu_seqlens, workspace, workspace_bytes, stream, w);
  if (st != DN_OK) return st;
  if (events && events[0] && hipEventRecord(events[0], stream) != hipSuccess) return DN_EHIP;

  // 1. forward sweep that stores every chunk-start state
  dn::FwdParams fp = fwd_params(s, q, k, v, beta, g, h0, cu_seqlens);
  fp.states = w.states;
  fp.chunk_base = w.chunk_base;
  fp.seq_order = w.order;
  if (recompute) {
    hipError_t e = s->chunk == 32 ? dn::launch_fwd_c32(fp, s->Dk, true, false, stream)
                                  : dn::launch_fwd(fp, s->dtype, s->Dk, true, false, stream);
    if (e != hipSuccess) return DN_EHIP;
  }
  if (events && events[1] && hipEventRecord(events[1], stream) != hipSuccess) return DN_EHIP;

  // 2. reverse sweep for the state gradients, 3. chunk-parallel token gradients
  dn::BwdParams bp = {};
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.dO = dO;
  bp.beta = beta;
  bp.g = g;
  bp.dhT = dhT;
  bp.cu = cu_seqlens;
  bp.chunk_base = w.chunk_base;
  bp.chunk_seq = w.chunk_seq;
  bp.seq_order = w.order;
  bp.states = w.states;
  bp.dstates = w.dstates;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.dbeta = dbeta;
  bp.dg = dg;
  bp.dh0 = dh0;
  bp.B = s->B;
  bp.T = s->T;
  bp.H = s->H;
  bp.DV = s->Dv;
  bp.N = s->n_seqs;
  bp.NC = fp.NC;
  bp.ntiles = s->Dv / 64;
  bp.xcd_map = fp.xcd_map;
  bp.total_chunks = (int)w.nchunks;
  bp.chunk = chunk_len(s);
  bp.q_in = pro.q_in;
  bp.k_in = pro.k_in;
  bp.x_in = pro.x_in;
  bp.gate_scale = pro.gate_scale;
  bp.beta_raw = pro.beta_raw;
  return from_hip(dn::launch_bwd(bp, s->dtype, s->Dk, stream, events ? events[2] : nullptr,
                                 events ? events[3] : nullptr));
}

}  // namespace

namespace dn {

dn_status bwd_recompute(const dn_shape *s, const void *q, const void *k, const void *v, const float *beta,
                        const float *g, const float *h0, const int32_t *cu_seqlens, const void *dO,
                        const float *dhT, float *dq, float *dk, float *dv, float *dbeta, float *dg, float *dh0,
                        void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_run(s, q, k, v, beta, g, h0, cu_seqlens, dO, dhT, dq, dk, dv, dbeta, dg, dh0, workspace,
                 workspace_bytes, stream, nullptr, true);
}

}  // namespace dn

extern "C" {

const char *dn_status_str(dn_status s) {
  switch (s) {
    case DN_OK: return "DN_OK";
    case DN_EINVAL: return "DN_EINVAL: invalid argument";
    case DN_EUNSUPPORTED: return "DN_EUNSUPPORTED: shape or dtype not supported";
    case DN_ENOWS: return "DN_ENOWS: workspace too small";
    case DN_EHIP: return "DN_EHIP: HIP launch error";
    case DN_ESCRATCH:
      return "DN_ESCRATCH: the shape needs more than the allocation-free entry point's static scratch buffer";
  }
  return "unknown dn_status";
}

size_t dn_chunk_fwd_workspace(const dn_shape *s) {
  if (!s || s->B <= 0 || s->n_seqs <= 0) return 0;
  return fwd_ws_bytes(s, s->n_seqs != s->B || s->B == 1);
}

dn_status dn_chunk_fwd(const dn_shape *s, const void *q, const void *k, const void *v,
                       const float *beta, const float *g, const float *h0,
                       const int32_t *cu_seqlens, void *o, float *hT, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  dn_status st = check_shape(s, cu_seqlens, true);
  if (st != DN_OK) return st;
  if (s->T > 0) {
    if (!q || !k || !v || !beta || !o) return DN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return DN_EINVAL;
  }
  const size_t need = cu_seqlens ? fwd_ws_bytes(s, true) : 0;
  if (need > 0 && (workspace_bytes < need || !workspace || !aligned16(workspace))) return DN_ENOWS;
  dn::FwdParams p = fwd_params(s, q, k, v, beta, g, h0, cu_seqlens);
  p.o = o;
  p.hT = hT;
  if (need > 0) {
    int32_t *order = static_cast<int32_t *>(workspace);
    if (dn::launch_seq_order(cu_seqlens, s->n_seqs, order, stream) != hipSuccess) return DN_EHIP;
    p.seq_order = order;
  }
  if (s->chunk == 32) return from_hip(dn::launch_fwd_c32(p, s->Dk, false, true, stream));
  return from_hip(dn::launch_fwd(p, s->dtype, s->Dk, false, true, stream));
}

size_t dn_chunk_bwd_workspace(const dn_shape *s) {
  if (!s || s->H <= 0 || s->Dk <= 0 || s->Dv <= 0 || s->B <= 0 || s->T < 0 || s->n_seqs <= 0)
    return 0;
  return bwd_layout(s, s->n_seqs != s->B || s->B == 1).total;
}

dn_status dn_chunk_bwd(const dn_shape *s, const void *q, const void *k, const void *v,
                       const float *beta, const float *g, const float *h0,
                       const int32_t *cu_seqlens, const void *dO, const float *dhT, float *dq,
                       float *dk, float *dv, float *dbeta, float *dg, float *dh0, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return dn_chunk_bwd_events(s, q, k, v, beta, g, h0, cu_seqlens, dO, dhT, dq, dk, dv, dbeta, dg, dh0,
                             workspace, workspace_bytes, stream, nullptr);
}

dn_status dn_chunk_bwd_events(const dn_shape *s, const void *q, const void *k, const void *v,
                              const float *beta, const float *g, const float *h0,
                              const int32_t *cu_seqlens, const void *dO, const float *dhT, float *dq,
                              float *dk, float *dv, float *dbeta, float *dg, float *dh0,
                              void *workspace, size_t workspace_bytes, hipStream_t stream,
                              hipEvent_t *events) {
  return bwd_run(s, q, k, v, beta, g, h0, cu_seqlens, dO, dhT, dq, dk, dv, dbeta, dg, dh0, workspace,
                 workspace_bytes, stream, events, true);
}

dn_status dn_chunk_fwd_save(const dn_shape *s, const void *q, const void *k, const void *v,
                            const float *beta, const float *g, const float *h0,
                            const int32_t *cu_seqlens, void *o, float *hT, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  dn_status st = check_train(s, cu_seqlens, q, k, v, beta);
  if (st != DN_OK) return st;
  if (s->T > 0 && (!o || !aligned16(o))) return DN_EINVAL;
  TrainWs w;
  st = train_ws(s, cu_seqlens, workspace, workspace_bytes, stream, w);
  if (st != DN_OK) return st;
  dn::FwdParams p = fwd_params(s, q, k, v, beta, g, h0, cu_seqlens);
  p.o = o;
  p.hT = hT;
  p.states = w.states;
  p.chunk_base = w.chunk_base;
  p.seq_order = w.order;
  if (s->chunk == 32) return from_hip(dn::launch_fwd_c32(p, s->Dk, true, true, stream));
  return from_hip(dn::launch_fwd(p, s->dtype, s->Dk, true, true, stream));
}

dn_status dn_chunk_bwd_saved(const dn_shape *s, const void *q, const void *k, const void *v,
                             const float *beta, const float *g, const float *h0,
                             const int32_t *cu_seqlens, const void *dO, const float *dhT, float *dq,
                             float *dk, float *dv, float *dbeta, float *dg, float *dh0, void *workspace,
                             size_t workspace_bytes, hipStream_t stream, hipEvent_t *events) {
  return bwd_run(s, q, k, v, beta, g, h0, cu_seqlens, dO, dhT, dq, dk, dv, dbeta, dg, dh0, workspace,
                 workspace_bytes, stream, events, false);
}

dn_status dn_chunk_bwd_prologue(const dn_shape *s, const void *q, const void *k, const void *v,
                                const float *beta, const float *g, const float *h0,
                                const int32_t *cu_seqlens, const void *dO, const float *dhT,
                                const void *q_in, const void *k_in, const float *x_in, float gate_scale,
                                float *dq_in, float *dk_in, float *dv, float *db_in, float *dx_in,
                                float *dh0, void *workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t *events) {
  if ((x_in == nullptr) != (g == nullptr)) return DN_EINVAL;
  if (s && s->chunk == 32) return DN_EUNSUPPORTED;  // the folded variants take 64-token chunks
  if (s && s->T > 0) {
    if (!q_in || !k_in || !aligned16(q_in) || !aligned16(k_in)) return DN_EINVAL;
  }
  ProIn pro;
  pro.q_in = q_in ? q_in : q;  // T == 0: nothing is read, but the variant is still the folded one
  pro.k_in = k_in ? k_in : k;
  pro.x_in = x_in;
  pro.gate_scale = gate_scale;
  return bwd_run(s, q, k, v, beta, g, h0, cu_seqlens, dO, dhT, dq_in, dk_in, dv, db_in, dx_in, dh0, workspace,
                 workspace_bytes, stream, events, false, pro);
}

dn_status dn_chunk_bwd_longhorn(const dn_shape *s, const void *q, const void *k, const void *v,
                                const float *eps, const float *g, const float *h0,
                                const int32_t *cu_seqlens, const void *dO, const float *dhT,
                                const float *beta, float *dq, float *dk, float *dv, float *dbeta, float *dg,
                                float *dh0, void *workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t *events) {
  if (s && s->chunk == 32) return DN_EUNSUPPORTED;  // the folded variants take 64-token chunks
  if (s && s->T > 0 && !beta) return DN_EINVAL;
  ProIn pro;
  pro.beta_raw = beta ? beta : eps;  // T == 0: nothing is read, but the variant is still the folded one
  return bwd_run(s, q, k, v, eps, g, h0, cu_seqlens, dO, dhT, dq, dk, dv, dbeta, dg, dh0, workspace,
                 workspace_bytes, stream, events, false, pro);
}

dn_status dn_recurrent_step(int32_t B, int32_t H, int32_t Dk, int32_t Dv, int32_t dtype,
                            const void *q, const void *k, const void *v, const float *beta,
                            const float *g, float *state, void *o, hipStream_t stream) {
  if (B <= 0 || H <= 0 || Dk <= 0 || Dv <= 0) return DN_EINVAL;
  if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
  if (Dk != 64 && Dk != 128) return DN_EUNSUPPORTED;
  if (Dv % 64 != 0 || Dv > 1024) return DN_EUNSUPPORTED;
  if (!q || !k || !v || !beta || !state || !o) return DN_EINVAL;
  if (!aligned16(state)) return DN_EINVAL;
  dn::StepParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.g = g;
  p.state = state;
  p.o = o;
  p.B = B;
  p.H = H;
  p.DV = Dv;
  return from_hip(dn::launch_step(p, dtype, Dk, stream));
}

static dn_status rows_check(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t dtype) {
  if (B <= 0 || T < 0 || H <= 0) return DN_EINVAL;
  if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
  if (Dk != 64 && Dk != 128) return DN_EUNSUPPORTED;
  // grid size: B T H / 4 rows of workgroups below 2^31 (B T checked first, so
  // that the product cannot overflow)
  const int64_t bt = (int64_t)B * T;
  if (bt > ((int64_t)1 << 33) / H || bt * H / 4 >= (int64_t)1 << 31) return DN_EUNSUPPORTED;
  return DN_OK;
}

dn_status dn_longhorn_eps(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t dtype, const void *k,
                          const float *beta, float *eps, hipStream_t stream) {
  dn_status st = rows_check(B, T, H, Dk, dtype);
  if (st != DN_OK) return st;
  const int64_t rows = (int64_t)B * T * H;
  if (rows == 0) return DN_OK;
  if (!k || !beta || !eps || !aligned16(k)) return DN_EINVAL;
  dn::LonghornParams p = {};
  p.k = k;
  p.beta = beta;
  p.eps = eps;
  p.rows = rows;
  return from_hip(dn::launch_longhorn(p, dtype, Dk, stream));
}

dn_status dn_longhorn_eps_bwd(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t dtype, const void *k,
                              const float *beta, const float *deps, float *dbeta, float *dk,
                              hipStream_t stream) {
  dn_status st = rows_check(B, T, H, Dk, dtype);
  if (st != DN_OK) return st;
  const int64_t rows = (int64_t)B * T * H;
  if (rows == 0) return DN_OK;
  if (!k || !beta || !deps || !dbeta || !dk || !aligned16(k) || !aligned16(dk)) return DN_EINVAL;
  dn::LonghornParams p = {};
  p.k = k;
  p.beta = beta;
  p.deps = deps;
  p.dbeta = dbeta;
  p.dk = dk;
  p.rows = rows;
  return from_hip(dn::launch_longhorn(p, dtype, Dk, stream));
}

dn_status dn_prologue(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t dtype, const void *q_in,
                      const void *k_in, const float *b_in, const float *x_in, float gate_scale, void *q,
                      void *k, float *beta, float *g, hipStream_t stream) {
  dn_status st = rows_check(B, T, H, Dk, dtype);
  if (st != DN_OK) return st;
  if ((x_in == nullptr) != (g == nullptr)) return DN_EINVAL;
  const int64_t rows = (int64_t)B * T * H;
  if (rows == 0) return DN_OK;
  if (!q_in || !k_in || !b_in || !q || !k || !beta) return DN_EINVAL;
  if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(q) || !aligned16(k)) return DN_EINVAL;
  dn::PrologueParams p = {};
  p.q_in = q_in;
  p.k_in = k_in;
  p.b_in = b_in;
  p.x_in = x_in;
  p.gate_scale = gate_scale;
  p.q = q;
  p.k = k;
  p.beta = beta;
  p.g = g;
  p.rows = rows;
  return from_hip(dn::launch_prologue(p, dtype, Dk, false, stream));
}

dn_status dn_prologue_bwd(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t dtype, const void *q_in,
                          const void *k_in, const float *b_in, const float *x_in, float gate_scale,
                          const float *dq, const float *dk, const float *dbeta, const float *dg,
                          float *dq_in, float *dk_in, float *db_in, float *dx_in, hipStream_t stream) {
  dn_status st = rows_check(B, T, H, Dk, dtype);
  if (st != DN_OK) return st;
  if ((x_in == nullptr) != (dg == nullptr) || (x_in == nullptr) != (dx_in == nullptr)) return DN_EINVAL;
  const int64_t rows = (int64_t)B * T * H;
  if (rows == 0) return DN_OK;
  if (!q_in || !k_in || !b_in || !dq || !dk || !dbeta || !dq_in || !dk_in || !db_in) return DN_EINVAL;
  if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(dq) || !aligned16(dk) || !aligned16(dq_in) ||
      !aligned16(dk_in))
    return DN_EINVAL;
  dn::PrologueParams p = {};
  p.q_in = q_in;
  p.k_in = k_in;
  p.b_in = b_in;
  p.x_in = x_in;
  p.gate_scale = gate_scale;
  p.dq = dq;
  p.dk = dk;
  p.dbeta = dbeta;
  p.dg = dg;
  p.dq_in = dq_in;
  p.dk_in = dk_in;
  p.db_in = db_in;
  p.dx_in = dx_in;
  p.rows = rows;
  return from_hip(dn::launch_prologue(p, dtype, Dk, true, stream));
}

static dn_status conv_check(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs,
                            int32_t dtype, const int32_t *cu_seqlens) {
  if (B <= 0 || T < 0 || H <= 0 || D <= 0) return DN_EINVAL;
  if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
  if (cu_seqlens ? (B != 1 || n_seqs < 1) : n_seqs != B) return DN_EINVAL;
  if (D % 8 != 0 || W < 1 || W > 4) return DN_EUNSUPPORTED;
  const int64_t C = (int64_t)H * D, TT = (int64_t)B * T;
  // grid: token blocks of 128 on x (< 2^31), channel groups of 512 on y (<= 65535)
  if ((C + 511) / 512 > 65535 || (TT + 127) / 128 >= ((int64_t)1 << 31)) return DN_EUNSUPPORTED;
  return DN_OK;
}

static dn::ConvParams conv_params(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs,
                                  const int32_t *cu_seqlens) {
  dn::ConvParams p = {};
  p.cu = cu_seqlens;
  p.TT = (int64_t)B * T;
  p.T = T;
  p.N = cu_seqlens ? n_seqs : B;
  p.C = H * D;
  p.W = W;
  return p;
}

dn_status dn_short_conv(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs, int32_t dtype,
                        const void *x, const float *w, const int32_t *cu_seqlens, void *y, hipStream_t stream) {
  const dn_status st = conv_check(B, T, H, D, W, n_seqs, dtype, cu_seqlens);
  if (st != DN_OK) return st;
  if ((int64_t)B * T == 0) return DN_OK;
  if (!x || !w || !y || !aligned16(x) || !aligned16(y)) return DN_EINVAL;
  dn::ConvParams p = conv_params(B, T, H, D, W, n_seqs, cu_seqlens);
  p.x = x;
  p.w = w;
  p.y = y;
  return from_hip(dn::launch_conv(p, dtype, false, stream));
}

dn_status dn_short_conv_bwd(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs,
                            int32_t dtype, const void *x, const float *w, const int32_t *cu_seqlens,
                            const float *dy, float *dx, float *dw, hipStream_t stream) {
  const dn_status st = conv_check(B, T, H, D, W, n_seqs, dtype, cu_seqlens);
  if (st != DN_OK) return st;
  if (!dw) return DN_EINVAL;
  const bool empty = (int64_t)B * T == 0;
  if (!empty && (!x || !w || !dy || !dx || !aligned16(x) || !aligned16(dy) || !aligned16(dx))) return DN_EINVAL;
  dn::ConvParams p = conv_params(B, T, H, D, W, n_seqs, cu_seqlens);
  p.x = x;
  p.w = w;
  p.dy = dy;
  p.dx = dx;
  p.dw = dw;
  return from_hip(dn::launch_conv(p, dtype, true, stream));
}

dn_status dn_short_conv_l2(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs,
                           int32_t dtype, const void *x, const float *w, const int32_t *cu_seqlens, void *y,
                           hipStream_t stream) {
  const dn_status st = conv_check(B, T, H, D, W, n_seqs, dtype, cu_seqlens);
  if (st != DN_OK) return st;
  if (D != 64 && D != 128) return DN_EUNSUPPORTED;
  if ((int64_t)B * T == 0) return DN_OK;
  if (!x || !w || !y || !aligned16(x) || !aligned16(y)) return DN_EINVAL;
  dn::ConvParams p = conv_params(B, T, H, D, W, n_seqs, cu_seqlens);
  p.x = x;
  p.w = w;
  p.y = y;
  p.norm_lanes = D / 8;
  return from_hip(dn::launch_conv(p, dtype, false, stream));
}

dn_status dn_short_conv_l2_bwd(int32_t B, int32_t T, int32_t H, int32_t D, int32_t W, int32_t n_seqs,
                               int32_t dtype, const void *x, const float *w, const int32_t *cu_seqlens,
                               const float *dy, float *dx, float *dw, hipStream_t stream) {
  const dn_status st = conv_check(B, T, H, D, W, n_seqs, dtype, cu_seqlens);
  if (st != DN_OK) return st;
  if (D != 64 && D != 128) return DN_EUNSUPPORTED;
  if (!dw) return DN_EINVAL;
  const bool empty = (int64_t)B * T == 0;
  if (!empty && (!x || !w || !dy || !dx || !aligned16(x) || !aligned16(dy) || !aligned16(dx))) return DN_EINVAL;
  dn::ConvParams p = conv_params(B, T, H, D, W, n_seqs, cu_seqlens);
  p.x = x;
  p.w = w;
  p.dy = dy;
  p.dx = dx;
  p.dw = dw;
  p.norm_lanes = D / 8;
  return from_hip(dn::launch_conv(p, dtype, true, stream));
}

}  // extern "C"
