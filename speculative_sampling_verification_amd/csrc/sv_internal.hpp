// Internal declarations shared by the kernels (sv_kernels.hip) and the C ABI (sv_abi.hip).
//
// Data flow of one spec_verify call (all on the caller's stream):
//   k_chunk   grid = rows x chunks : streams every logit once; per chunk a max and a sum of
//                                     exponentials (or an argmax when greedy)
//   k_row     grid = rows          : merges the chunks of a row into its distribution
//                                     parameters (max m, threshold thr, normaliser S)
//   k_seq     grid = B             : accept tests, first-rejection scan, and the final draw when
//                                     the final row is greedy
//   k_final_partial / k_final_pick : the final draw over a full row pair (top-p: or over the
//                                     kept segments k_topp_cand wrote for the target row)
// With compact top-k rows (top-k <= kCompactMaxK) two launches do everything: k_topk_row (one
// workgroup per row: streaming, candidate selection and the row merge) and k_seq_compact (one
// workgroup per sequence: accept tests and the final draw).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "spec_verify.h"

namespace sv {

constexpr int kThreads = 256;        // threads per workgroup of the streaming kernels (4 waves)
constexpr int kVecPerThread = 16;    // 16-byte vectors each thread holds per chunk
constexpr int kCompactMaxK = 256;    // top-k <= this uses the compact candidate path
constexpr int kKeptCap = 1024;       // kept tokens a compact row may hold
constexpr int kSeqThreads = 64;      // one wave per sequence
constexpr int kHistBins = 512;       // top-p mass histogram bins per chunk (bf16) ...
constexpr int kHistPerUnit = 8;      // ... on a grid of 1/8 of a unit of z / T
constexpr int kHistBinsF32 = 256;    // fp32 rows: as many as the edge codes resolve (the last
                                     // bin, like code kCodeFar, holds everything lower)
// Histogram bins per chunk for logits of esize bytes.
inline int hist_bins(int esize) { return esize == 4 ? kHistBinsF32 : kHistBins; }
constexpr int kTopPCandCap = 4096;   // boundary candidates a top-p row may hold
constexpr int kTopPSegCap = 1024;    // kept-list entries of one chunk of a top-p target row
constexpr int kMentorBisectionSteps = 50;  // bisection steps on alpha (mentored decoding)
constexpr int kRestMaxM = 128;  // candidates per sequence (REST tree builder)
constexpr int kRestMaxL = 32;   // tokens per candidate
constexpr int kRestMaxN = 256;  // tree nodes, root included
constexpr int64_t kPhiloxMaxN = (int64_t)1 << 40;  // uniforms per spec_philox_uniform call
constexpr size_t kNoAllocScratchBytes = SPEC_VERIFY_NOALLOC_SCRATCH_BYTES;  // spec_verify_noalloc

// Row kinds written by k_row.
enum RowKind : int { kRowDense = 0, kRowCompact = 1, kRowGreedy = 2 };

struct alignas(16) ChunkPart {
  float vmax;      // largest logit of the chunk
  int argmax;      // lowest index holding vmax (k_chunk_argmax), else -1
  double sum;      // sum of exp((z - vmax) / T) over the chunk (dense mode), else 0
  int pad[4];
};

struct alignas(16) RowStat {
  float m;         // largest logit of the row
  float thr;       // kept tokens are those with z >= thr (-inf: all)
  double S;        // sum over kept tokens of exp((z - m) / T)
  int argmax;      // lowest index of the maximum (greedy rows)
  int nkept;       // number of kept tokens (compact rows), else -1
  int kind;        // RowKind
  int pad;
};

// Top-p selection state of a row (histogram path): the boundary lies among the elements whose
// grid edge floor(8 z / T) is in [e_lo, e_hi]; every element above e_hi is kept.
struct alignas(16) TopPRow {
  double mass_above;  // sum of exp((z - m) / T) over the elements above e_hi
  int e_lo, e_hi;     // candidate edge range (e_lo = INT_MIN: open below)
  int count;          // candidates appended (may exceed kTopPCandCap: the row falls back)
  int coded;          // 1: the row's edge codes resolve [e_lo, e_hi] (the candidate pass reads
                      // the codes instead of the logits)
  int em;             // the grid edge of the row maximum
  int pad[3];
};

// Edge codes (fp32 top-p rows): one byte per element of a chunk frame, the element's grid edge
// below its chunk's top edge, etop - floor(8 z / T), or kCodeFar when that is kCodeFar or more
// (or the element is -inf, or outside the row).
constexpr int kCodeFar = 255;

// How a draft position is decided under mentored decoding.
enum MentorMode : int {
  kMentorLossless = 0,  // a row of the pair has no kept list: the lossless rule
  kMentorShortcut = 1,  // u < min(1, q/p): accepted without solving (r is never smaller)
  kMentorTrivial = 2,   // KL(q || p) <= D: every draft token with p > 0 is accepted
  kMentorSolved = 3,    // alpha and beta solved
  kMentorDeferred = 4   // kept list longer than k_mentor holds: solved in k_seq_compact
};

// Per-position result of the mentored solve (k_mentor), read by the accept scan and the draw.
struct alignas(16) MentorSol {
  double a;           // accept probability of the draft token
  double qx, px;      // q and p of the draft token (fp64 normalisers below)
  double alpha, beta; // solved parameters (kMentorSolved; beta = inf: no replacement mass)
  double st, sd;      // sum over the target / draft kept set of exp(z/T - m/T), in fp64
  int mode;           // MentorMode
  int pad;
};

struct alignas(16) SeqState {
  int n;           // accepted drafts
  int need_dense;  // 1 if the final draw runs in k_final_partial / k_final_pick
  int fallback;    // 1 if the residual had zero mass and q was used
  int need_list;   // 1 if the final draw runs over the target row's kept segments (top-p)
};

struct Dims {
  int B, K, V;
  int draft_rows;   // rows per sequence in the draft tensor
  int rows_per_seq; // 2K+1 for verify, 1 for plain row sets
  int rows;         // total rows
  int chunk_elems;  // elements per chunk
  int nchunks;      // chunks per row
  int vec;          // 1: 16-byte loads are legal for every row
  int fchunk_elems; // elements per chunk of the final draw (a chunk, or one vector row of it)
  int nfchunks;     // final-draw chunks per row, counted from the row's first element
  int esize;        // bytes per logit (2: bf16, 4: fp32)
};

struct Samp {
  float temperature;
  float inv_t;      // 1 / temperature (0 when greedy)
  int top_k;        // effective top-k (0 = off)
  float top_p;      // effective top-p (1 = off)
  float lenience;
  int greedy;       // temperature == 0
  int compact;      // compact top-k path
  int generic_trunc;// truncation that needs the row-pass selection (top-k > kCompactMaxK or top-p
                    // without a compact list)
  int topp_hist;    // top-p without top-k: histogram, boundary candidates, exact selection
  int mentor;       // mentored decoding (KL bound > 0, compact rows, K > 0)
  double mentor_d;  // the KL bound D
};

struct Workspace {
  ChunkPart* parts;  // [rows][nchunks]
  RowStat* rstat;    // [rows]
  uint2* kept;       // [rows][kKeptCap]  (index, float bits)      compact only
  SeqState* seq;     // [B]
  double2* fpart;    // [B][nfchunks]  (residual mass, target mass)
  RowStat* dstat;    // [B][2] statistics of the final draw's rows (target; draft, or the
                     // target again for the bonus draw)
  int32_t* nbuf;     // [B] accepted counts when the caller does not want them
  unsigned long long* hist;  // [rows][nchunks][hist_bins] fixed-point mass   top-p histogram only
  TopPRow* tprow;            // [rows]                                        top-p histogram only
  uint2* tcand;              // [rows][kTopPCandCap] (index, bits)            top-p bf16 only
  uint32_t* tkept;           // [B*(K+1)][nchunks][kTopPSegCap] index of every element of a
                             // target row's chunk at or above the boundary bracket, in no
                             // particular order                             top-p histogram only
  int* tkcnt;                // [B*(K+1)][nchunks] entries of each segment (> kTopPSegCap:
                             // overflowed)                                   top-p histogram only
  ulonglong2* lpart;         // [B][nchunks] the final draw's fixed-point masses (residual, q) of
                             // each segment                                  top-p histogram only
  uint8_t* codes;            // [rows][nchunks * chunk_elems] edge codes     top-p fp32 only
  MentorSol* ment;           // [B][K]                                        mentored only
  double* bpart;             // [B*K][nfchunks] acceptance-rate partials      dense rows only
};

inline int chunk_elems_for(sv_dtype dt) {
  return kThreads * kVecPerThread * (dt == SV_DTYPE_BF16 ? 8 : 4);
}

// Top-p rows carry edge codes when a code (one byte) is smaller than the logit: fp32.
inline bool topp_codes(const Dims& d, const Samp& s) { return s.topp_hist && d.esize == 4; }

// Workspace layout; returns the byte size and, when base != nullptr, fills ws.
size_t layout_verify(const Dims& d, const Samp& s, void* base, Workspace* ws);
size_t layout_tree(const Dims& d, void* base, Workspace* ws);

// Kernel launchers (sv_kernels.hip).  Return hipSuccess or the launch error.
hipError_t launch_verify(const void* target, const void* draft, sv_dtype dt, const Dims& d,
                         const Samp& s, const int32_t* drafts, const float* uniforms,
                         int32_t* out_tokens, int32_t* out_n, float* out_a, float* out_q,
                         float* out_p, float* out_beta, bool rates_only, const Workspace& ws,
                         hipStream_t stream, hipEvent_t* events, int n_events,
                         const Workspace* presampled = nullptr);
hipError_t launch_philox_uniform(uint64_t key0, uint64_t key1, uint64_t counter, int64_t n,
                                 float* out, hipStream_t stream);
hipError_t launch_rest_tree(const int32_t* cands, int B, int M, int L, int N, int32_t* parent,
                            int32_t* tokens, int32_t* n_nodes, int32_t* depth, int32_t* weight,
                            uint8_t* mask, hipStream_t stream);
hipError_t launch_tree(const void* target, sv_dtype dt, const Dims& d, const int32_t* parent,
                       const int32_t* tokens, int max_depth, int32_t* out_tokens,
                       int32_t* out_n, int32_t* out_last, const Workspace& ws,
                       hipStream_t stream, hipEvent_t* events, int n_events);

}  // namespace sv
