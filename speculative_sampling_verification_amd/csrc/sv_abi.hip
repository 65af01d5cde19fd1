// extern "C" entry points of libspecverify.so: host-side argument checks, workspace layout and
// kernel dispatch.  No allocation, no synchronisation; everything is enqueued on the caller's
// stream.  See include/spec_verify.h for the contract of each function.

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "sv_internal.hpp"

// Scratch memory of spec_verify_noalloc, for callers that cannot allocate: one copy of this
// array per GPU, held from the library's load until the process ends.  Host code never uses
// its name as an address (on the host it is only a stand-in for the device symbol): the device
// address comes from hipGetSymbolAddress, once per device, in noalloc_scratch() below.
static __device__ __align__(256) unsigned char scratch[sv::kNoAllocScratchBytes];

namespace sv {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Appends a segment of `bytes` to the layout; returns its offset.
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

template <class T>
T* at(void* base, size_t off) {
  return base ? reinterpret_cast<T*>(static_cast<char*>(base) + off) : nullptr;
}

bool valid_dtype(sv_dtype dt) { return dt == SV_DTYPE_F32 || dt == SV_DTYPE_BF16; }
size_t esize(sv_dtype dt) { return dt == SV_DTYPE_BF16 ? 2 : 4; }

bool valid_params(const sv_sampling* p) {
  if (!p) return false;
  if (!(p->temperature >= 0.0f) || !std::isfinite(p->temperature)) return false;
  if (p->top_k < 0) return false;
  if (!(p->top_p > 0.0f && p->top_p <= 1.0f)) return false;
  if (!(p->lenience > 0.0f && p->lenience <= 1.0f)) return false;
  if (!(p->mentor_kl >= 0.0f) || !std::isfinite(p->mentor_kl)) return false;
  return true;
}

Samp make_samp(const sv_sampling* p, int V);

// Mentored decoding with draft tokens to verify needs the lossless comparison (lenience 1) and,
// for sampled rows, the compact top-k lists.
bool valid_mentor(const sv_sampling* p, int V, int K) {
  if (p->mentor_kl == 0.0f || K == 0) return true;
  if (p->lenience != 1.0f) return false;
  const Samp s = make_samp(p, V);
  return s.greedy || s.compact;
}

Samp make_samp(const sv_sampling* p, int V) {
  Samp s{};
  s.temperature = p->temperature;
  s.greedy = p->temperature == 0.0f;
  s.inv_t = s.greedy ? 0.0f : 1.0f / p->temperature;
  s.top_k = (p->top_k > 0 && p->top_k < V) ? p->top_k : 0;
  s.top_p = p->top_p;
  s.lenience = p->lenience;
  s.compact = !s.greedy && s.top_k > 0 && s.top_k <= kCompactMaxK;
  s.generic_trunc = !s.greedy && ((s.top_k > kCompactMaxK) || (s.top_p < 1.0f && !s.compact));
  s.topp_hist = !s.greedy && s.top_k == 0 && s.top_p < 1.0f;
  s.mentor_d = (double)p->mentor_kl;
  s.mentor = s.compact && p->mentor_kl > 0.0f;  // greedy rows: the lossless rule is the optimum
  return s;
}

// Fills Dims for a verify-shaped problem; false if the sizes do not fit the indexing.
bool make_dims(int B, int K, int V, int draft_rows, sv_dtype dt, Dims* d) {
  if (B < 1 || K < 0 || V < 1) return false;
  const long long rps = 2LL * K + 1;
  const long long rows = (long long)B * rps;
  if (rows > INT_MAX) return false;
  const int ce = chunk_elems_for(dt);
  // chunks of a row counted from the 16-byte boundary at or before its start (the chunked
  // kernels' frame): up to EPV - 1 more elements than V; set_alignment narrows it to V's
  // chunks when every row is aligned
  const int epv = 16 / (int)esize(dt);
  const long long nch = ((long long)V + epv - 1 + ce - 1) / ce;
  if (rows * nch > (long long)INT_MAX) return false;
  if ((long long)B * nch > (long long)INT_MAX) return false;
  d->B = B;
  d->K = K;
  d->V = V;
  d->draft_rows = draft_rows;
  d->rows_per_seq = (int)rps;
  d->rows = (int)rows;
  d->chunk_elems = ce;
  d->nchunks = (int)nch;
  d->vec = 0;
  d->esize = (int)esize(dt);
  // the final draw runs one workgroup per (sequence, final chunk): one vector row of a chunk
  // when whole chunks would leave most of the 256 CUs idle, a quarter chunk (several rounds
  // of short workgroups) up to 64 K workgroups, else whole chunks
  const long long bn = (long long)B * nch;
  const int fce = bn < 1024 ? ce / kVecPerThread : bn < 16384 ? ce / 4 : ce;
  d->fchunk_elems = fce;
  d->nfchunks = (int)(((long long)V + fce - 1) / fce);
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Records whether every row starts on a 16-byte boundary (16-byte loads in every kernel) and
// then counts the chunks of V alone.
void set_alignment(Dims* d, bool aligned) {
  d->vec = aligned ? 1 : 0;
  if (aligned) d->nchunks = (d->V + d->chunk_elems - 1) / d->chunk_elems;
}

// Logit pointers must be aligned to their element size (any 16-byte phase is handled).
bool elem_aligned(const void* p, sv_dtype dt) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % esize(dt)) == 0;
}

}  // namespace

size_t layout_verify(const Dims& d, const Samp& s, void* base, Workspace* ws) {
  Carver c;
  const size_t rows = (size_t)d.rows, nch = (size_t)d.nchunks;
  const size_t o_parts = c.take(s.compact ? 0 : rows * nch * sizeof(ChunkPart));
  const size_t o_rstat = c.take(rows * sizeof(RowStat));
  const size_t o_kept = c.take(s.compact ? rows * kKeptCap * sizeof(uint2) : 0);
  const size_t o_seq = c.take((size_t)d.B * sizeof(SeqState));
  const size_t o_fpart = c.take(s.greedy ? 0 : (size_t)d.B * d.nfchunks * sizeof(double2));
  const size_t o_dstat = c.take(s.greedy ? 0 : (size_t)d.B * 2 * sizeof(RowStat));
  const size_t o_n = c.take((size_t)d.B * sizeof(int32_t));
  const bool th = s.topp_hist != 0;
  const size_t o_hist =
      c.take(th ? rows * nch * hist_bins(d.esize) * sizeof(unsigned long long) : 0);
  const size_t o_tprow = c.take(th ? rows * sizeof(TopPRow) : 0);
  const bool cd = topp_codes(d, s);  // fp32: candidates kept in LDS, edge codes instead
  const size_t o_tcand = c.take(th && !cd ? rows * kTopPCandCap * sizeof(uint2) : 0);
  const size_t tsegs = th && !cd ? (size_t)d.B * (d.K + 1) * nch : 0;  // bf16 kept segments
  const size_t o_tkept = c.take(tsegs * kTopPSegCap * sizeof(uint32_t));
  const size_t o_tkcnt = c.take(tsegs * sizeof(int));
  const size_t o_lpart = c.take(th ? (size_t)d.B * nch * sizeof(ulonglong2) : 0);
  const size_t o_codes = c.take(cd ? rows * nch * (size_t)d.chunk_elems : 0);
  const bool me = s.mentor && d.K > 0;
  const size_t o_ment = c.take(me ? (size_t)d.B * d.K * sizeof(MentorSol) : 0);
  const bool bp = !s.compact && !s.greedy;
  const size_t o_bpart = c.take(bp ? (size_t)d.B * d.K * d.nfchunks * sizeof(double) : 0);
  if (ws) {
    ws->parts = s.compact ? nullptr : at<ChunkPart>(base, o_parts);
    ws->rstat = at<RowStat>(base, o_rstat);
    ws->kept = s.compact ? at<uint2>(base, o_kept) : nullptr;
    ws->seq = at<SeqState>(base, o_seq);
    ws->fpart = s.greedy ? nullptr : at<double2>(base, o_fpart);
    ws->dstat = s.greedy ? nullptr : at<RowStat>(base, o_dstat);
    ws->nbuf = at<int32_t>(base, o_n);
    ws->hist = th ? at<unsigned long long>(base, o_hist) : nullptr;
    ws->tprow = th ? at<TopPRow>(base, o_tprow) : nullptr;
    ws->tcand = th && !cd ? at<uint2>(base, o_tcand) : nullptr;
    ws->tkept = tsegs ? at<uint32_t>(base, o_tkept) : nullptr;
    ws->tkcnt = tsegs ? at<int>(base, o_tkcnt) : nullptr;
    ws->lpart = th ? at<ulonglong2>(base, o_lpart) : nullptr;
    ws->codes = cd ? at<uint8_t>(base, o_codes) : nullptr;
    ws->ment = me ? at<MentorSol>(base, o_ment) : nullptr;
    ws->bpart = bp ? at<double>(base, o_bpart) : nullptr;
  }
  return c.off;
}

size_t layout_tree(const Dims& d, void* base, Workspace* ws) {
  Carver c;
  const size_t o_parts = c.take((size_t)d.rows * d.nchunks * sizeof(ChunkPart));
  if (ws) {
    *ws = Workspace{};
    ws->parts = at<ChunkPart>(base, o_parts);
  }
  return c.off;
}

}  // namespace sv

using namespace sv;

namespace {

// Device address of the scratch array on the GPU that `stream` belongs to (the current device
// for the null stream), looked up with that device current on the first call for the device
// and kept per device.  SV_ERR_LAUNCH if a HIP query fails.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

int noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  const hipError_t ed = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (ed != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_LAUNCH;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) return SV_ERR_LAUNCH;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return SV_ERR_LAUNCH;
      void* q = nullptr;
      const hipError_t eg = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (cur != dev) (void)hipSetDevice(cur);
      if (eg != hipSuccess || q == nullptr) return SV_ERR_LAUNCH;
      g_scratch_ptr[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return SV_OK;
}

int verify_impl(const void* target, const void* draft, sv_dtype dtype, int B, int K, int V,
                int draft_rows, const int32_t* drafts, const float* uniforms,
                const sv_sampling* params, int32_t* out_tokens, int32_t* out_n, float* out_a,
                float* out_q, float* out_p, float* out_beta, void* workspace,
                size_t workspace_bytes, hipStream_t stream, hipEvent_t* events, int n_events,
                const void* sample_ws = nullptr, size_t sample_ws_bytes = 0,
                bool use_scratch = false) {
  if (!valid_dtype(dtype)) return SV_ERR_UNSUPPORTED_DTYPE;
  if (!valid_params(params)) return SV_ERR_INVALID_ARG;
  if (K > 0 && draft_rows != K && draft_rows != K + 1) return SV_ERR_INVALID_ARG;
  if (V < 1 || !valid_mentor(params, V, K)) return SV_ERR_INVALID_ARG;
  Dims d{};
  if (!make_dims(B, K, V, K > 0 ? draft_rows : 0, dtype, &d)) return SV_ERR_INVALID_ARG;
  if (!target || !uniforms || !out_tokens) return SV_ERR_INVALID_ARG;
  if (K > 0 && (!draft || !drafts)) return SV_ERR_INVALID_ARG;
  if (!elem_aligned(target, dtype) || (K > 0 && !elem_aligned(draft, dtype)))
    return SV_ERR_INVALID_ARG;
  if (events && n_events < 2) return SV_ERR_INVALID_ARG;
  const Samp s = make_samp(params, V);
  // draft rows summarised by an earlier spec_sample over them (rows b*K + k there)
  if (sample_ws && (K < 1 || draft_rows != K || !s.compact)) return SV_ERR_INVALID_ARG;
  const size_t need = layout_verify(d, s, nullptr, nullptr);
  if (use_scratch) {  // spec_verify_noalloc: the library's scratch array is the workspace
    if (need > kNoAllocScratchBytes) return SV_ERR_SCRATCH_TOO_SMALL;
    const int st = noalloc_scratch(stream, &workspace);
    if (st != SV_OK) return st;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (!workspace || workspace_bytes < need) return SV_ERR_WORKSPACE_TOO_SMALL;
  Workspace ws_s{};
  if (sample_ws) {
    Dims ds{};
    if (!make_dims(B * K, 0, V, 0, dtype, &ds)) return SV_ERR_INVALID_ARG;
    if (sample_ws_bytes < layout_verify(ds, s, nullptr, nullptr))
      return SV_ERR_WORKSPACE_TOO_SMALL;
    layout_verify(ds, s, const_cast<void*>(sample_ws), &ws_s);
  }
  set_alignment(&d, ((size_t)V * esize(dtype)) % 16 == 0 && aligned16(target) &&
                        (K == 0 || aligned16(draft)));
  Workspace ws{};
  layout_verify(d, s, workspace, &ws);
  if (!out_n) out_n = ws.nbuf;
  const hipError_t e = launch_verify(target, draft, dtype, d, s, drafts, uniforms, out_tokens,
                                     out_n, out_a, out_q, out_p, out_beta, false, ws, stream,
                                     events, n_events, sample_ws ? &ws_s : nullptr);
  return e == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int B, int K, int V, sv_dtype dtype, const sv_sampling* params) {
  if (!valid_dtype(dtype) || !valid_params(params)) return 0;
  if (V < 1 || K < 0 || !valid_mentor(params, V, K)) return 0;
  Dims d{};
  if (!make_dims(B, K, V, K, dtype, &d)) return 0;
  return layout_verify(d, make_samp(params, V), nullptr, nullptr);
}

int spec_verify(const void* target_logits, const void* draft_logits, sv_dtype dtype, int B, int K,
                int V, int draft_rows, const int32_t* draft_tokens, const float* uniforms,
                const sv_sampling* params, int32_t* out_tokens, int32_t* out_num_accepted,
                float* out_accept_prob, float* out_q_draft, float* out_p_draft, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  if (!out_num_accepted) return SV_ERR_INVALID_ARG;
  return verify_impl(target_logits, draft_logits, dtype, B, K, V, draft_rows, draft_tokens,
                     uniforms, params, out_tokens, out_num_accepted, out_accept_prob,
                     out_q_draft, out_p_draft, nullptr, workspace, workspace_bytes, stream,
                     nullptr, 0);
}

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                        int B, int K, int V, int draft_rows, const int32_t* draft_tokens,
                        const float* uniforms, const sv_sampling* params, int32_t* out_tokens,
                        int32_t* out_num_accepted, float* out_accept_prob, float* out_q_draft,
                        float* out_p_draft, hipStream_t stream) {
  if (!out_num_accepted) return SV_ERR_INVALID_ARG;
  return verify_impl(target_logits, draft_logits, dtype, B, K, V, draft_rows, draft_tokens,
                     uniforms, params, out_tokens, out_num_accepted, out_accept_prob,
                     out_q_draft, out_p_draft, nullptr, nullptr, 0, stream, nullptr, 0, nullptr,
                     0, true);
}

int spec_verify_presampled(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                           int B, int K, int V, const int32_t* draft_tokens,
                           const float* uniforms, const sv_sampling* params,
                           int32_t* out_tokens, int32_t* out_num_accepted,
                           float* out_accept_prob, float* out_q_draft, float* out_p_draft,
                           const void* sample_workspace, size_t sample_workspace_bytes,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!out_num_accepted || !sample_workspace) return SV_ERR_INVALID_ARG;
  return verify_impl(target_logits, draft_logits, dtype, B, K, V, K, draft_tokens, uniforms,
                     params, out_tokens, out_num_accepted, out_accept_prob, out_q_draft,
                     out_p_draft, nullptr, workspace, workspace_bytes, stream, nullptr, 0,
                     sample_workspace, sample_workspace_bytes);
}

int spec_verify_rates(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                      int B, int K, int V, int draft_rows, const int32_t* draft_tokens,
                      const float* uniforms, const sv_sampling* params, int32_t* out_tokens,
                      int32_t* out_num_accepted, float* out_accept_prob, float* out_q_draft,
                      float* out_p_draft, float* out_beta, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (!out_num_accepted || !out_beta || K < 1) return SV_ERR_INVALID_ARG;
  if (params && params->mentor_kl != 0.0f) return SV_ERR_INVALID_ARG;
  return verify_impl(target_logits, draft_logits, dtype, B, K, V, draft_rows, draft_tokens,
                     uniforms, params, out_tokens, out_num_accepted, out_accept_prob,
                     out_q_draft, out_p_draft, out_beta, workspace, workspace_bytes, stream,
                     nullptr, 0);
}

int spec_verify_profiled(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                         int B, int K, int V, int draft_rows, const int32_t* draft_tokens,
                         const float* uniforms, const sv_sampling* params, int32_t* out_tokens,
                         int32_t* out_num_accepted, float* out_accept_prob, float* out_q_draft,
                         float* out_p_draft, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, hipEvent_t* events, int n_events) {
  if (!out_num_accepted || !events || n_events < 2) return SV_ERR_INVALID_ARG;
  return verify_impl(target_logits, draft_logits, dtype, B, K, V, draft_rows, draft_tokens,
                     uniforms, params, out_tokens, out_num_accepted, out_accept_prob,
                     out_q_draft, out_p_draft, nullptr, workspace, workspace_bytes, stream, events,
                     n_events);
}

size_t spec_sample_workspace_size(int R, int V, sv_dtype dtype, const sv_sampling* params) {
  return spec_verify_workspace_size(R, 0, V, dtype, params);
}

int spec_sample(const void* logits, sv_dtype dtype, int R, int V, const float* uniforms,
                const sv_sampling* params, int32_t* out_tokens, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  return verify_impl(logits, nullptr, dtype, R, 0, V, 0, nullptr, uniforms, params, out_tokens,
                     nullptr, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes,
                     stream, nullptr, 0);
}

size_t spec_verify_tree_workspace_size(int B, int N, int V, sv_dtype dtype) {
  if (!valid_dtype(dtype) || B < 1 || N < 1 || N > 2048) return 0;
  if ((long long)B * N > INT_MAX) return 0;
  Dims d{};
  if (!make_dims(B * N, 0, V, 0, dtype, &d)) return 0;
  return layout_tree(d, nullptr, nullptr);
}

namespace {
int tree_impl(const void* target_logits, sv_dtype dtype, int B, int N, int V,
              const int32_t* parent, const int32_t* node_tokens, int max_depth,
              int32_t* out_tokens, int32_t* out_num_accepted, int32_t* out_last_node,
              void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
              int n_events) {
  if (!valid_dtype(dtype)) return SV_ERR_UNSUPPORTED_DTYPE;
  if (B < 1 || N < 1 || N > 2048 || V < 1 || max_depth < 0) return SV_ERR_INVALID_ARG;
  if ((long long)B * N > INT_MAX) return SV_ERR_INVALID_ARG;
  if (!target_logits || !parent || !node_tokens || !out_tokens || !out_num_accepted)
    return SV_ERR_INVALID_ARG;
  if (!elem_aligned(target_logits, dtype)) return SV_ERR_INVALID_ARG;
  Dims d{};
  if (!make_dims(B * N, 0, V, 0, dtype, &d)) return SV_ERR_INVALID_ARG;
  const size_t need = layout_tree(d, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return SV_ERR_WORKSPACE_TOO_SMALL;
  set_alignment(&d, ((size_t)V * esize(dtype)) % 16 == 0 && aligned16(target_logits));
  Workspace ws{};
  layout_tree(d, workspace, &ws);
  // the walk kernel reads B and the node count from Dims
  d.B = B;
  d.K = N;
  const hipError_t e = launch_tree(target_logits, dtype, d, parent, node_tokens, max_depth,
                                   out_tokens, out_num_accepted, out_last_node, ws, stream,
                                   events, n_events);
  return e == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
}  // namespace

int spec_verify_tree(const void* target_logits, sv_dtype dtype, int B, int N, int V,
                     const int32_t* parent, const int32_t* node_tokens, int max_depth,
                     int32_t* out_tokens, int32_t* out_num_accepted, int32_t* out_last_node,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return tree_impl(target_logits, dtype, B, N, V, parent, node_tokens, max_depth, out_tokens,
                   out_num_accepted, out_last_node, workspace, workspace_bytes, stream, nullptr,
                   0);
}

int spec_verify_tree_profiled(const void* target_logits, sv_dtype dtype, int B, int N, int V,
                              const int32_t* parent, const int32_t* node_tokens, int max_depth,
                              int32_t* out_tokens, int32_t* out_num_accepted,
                              int32_t* out_last_node, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, hipEvent_t* events, int n_events) {
  if (!events || n_events < 2) return SV_ERR_INVALID_ARG;
  return tree_impl(target_logits, dtype, B, N, V, parent, node_tokens, max_depth, out_tokens,
                   out_num_accepted, out_last_node, workspace, workspace_bytes, stream, events,
                   n_events);
}

int spec_acceptance_rate(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                         int B, int K, int V, int draft_rows, const sv_sampling* params,
                         float* out_beta, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (!valid_dtype(dtype)) return SV_ERR_UNSUPPORTED_DTYPE;
  if (!valid_params(params) || params->mentor_kl != 0.0f) return SV_ERR_INVALID_ARG;
  if (K < 1 || (draft_rows != K && draft_rows != K + 1)) return SV_ERR_INVALID_ARG;
  if (!target_logits || !draft_logits || !out_beta) return SV_ERR_INVALID_ARG;
  if (!elem_aligned(target_logits, dtype) || !elem_aligned(draft_logits, dtype))
    return SV_ERR_INVALID_ARG;
  Dims d{};
  if (!make_dims(B, K, V, draft_rows, dtype, &d)) return SV_ERR_INVALID_ARG;
  const Samp s = make_samp(params, V);
  const size_t need = layout_verify(d, s, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return SV_ERR_WORKSPACE_TOO_SMALL;
  set_alignment(&d, ((size_t)V * esize(dtype)) % 16 == 0 && aligned16(target_logits) &&
                        aligned16(draft_logits));
  Workspace ws{};
  layout_verify(d, s, workspace, &ws);
  const hipError_t e = launch_verify(target_logits, draft_logits, dtype, d, s, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, nullptr, nullptr, out_beta, true,
                                     ws, stream, nullptr, 0);
  return e == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

double spec_expected_tokens(double alpha, int gamma) {
  if (!(alpha >= 0.0 && alpha <= 1.0) || gamma < 0) return NAN;
  if (alpha == 1.0) return (double)gamma + 1.0;
  return (1.0 - std::pow(alpha, (double)gamma + 1.0)) / (1.0 - alpha);
}

double spec_walltime_speedup(double alpha, int gamma, double c) {
  if (!(c >= 0.0)) return NAN;
  return spec_expected_tokens(alpha, gamma) / ((double)gamma * c + 1.0);
}

double spec_ops_factor(double alpha, int gamma, double c_hat) {
  if (!(c_hat >= 0.0)) return NAN;
  return ((double)gamma * c_hat + (double)gamma + 1.0) / spec_expected_tokens(alpha, gamma);
}

int spec_optimal_gamma(double alpha, double c, int max_gamma) {
  if (!(alpha >= 0.0 && alpha <= 1.0) || !(c >= 0.0) || max_gamma < 1) return -1;
  int best_g = 1;
  double best = -INFINITY;
  for (int g = 1; g <= max_gamma; ++g) {
    const double v = spec_walltime_speedup(alpha, g, c);
    if (v > best) {
      best = v;
      best_g = g;
    }
  }
  return best_g;
}

int spec_build_tree(const int32_t* candidates, int B, int M, int L, int N, int32_t* out_parent,
                    int32_t* out_tokens, int32_t* out_num_nodes, int32_t* out_depth,
                    int32_t* out_weight, uint8_t* out_mask, hipStream_t stream) {
  if (B < 1 || M < 1 || M > kRestMaxM || L < 1 || L > kRestMaxL || N < 1 || N > kRestMaxN)
    return SV_ERR_INVALID_ARG;
  if ((long long)B * M * L > INT_MAX || (long long)B * N * N > INT_MAX) return SV_ERR_INVALID_ARG;
  if (!candidates || !out_parent || !out_tokens || !out_num_nodes) return SV_ERR_INVALID_ARG;
  const hipError_t e = launch_rest_tree(candidates, B, M, L, N, out_parent, out_tokens,
                                        out_num_nodes, out_depth, out_weight, out_mask, stream);
  return e == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

int spec_philox_uniform(uint64_t key0, uint64_t key1, uint64_t counter, int64_t n, float* out,
                        hipStream_t stream) {
  if (n < 0 || n > kPhiloxMaxN || (n > 0 && !out)) return SV_ERR_INVALID_ARG;
  if (n == 0) return SV_OK;
  const hipError_t e = launch_philox_uniform(key0, key1, counter, n, out, stream);
  return e == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case SV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SV_ERR_LAUNCH: return "kernel launch failed";
    case SV_ERR_SCRATCH_TOO_SMALL:
      return "problem needs more than spec_verify_noalloc's built-in scratch buffer";
    default: return "unknown status";
  }
}

}  // extern "C"
