// REST draft-tree construction on gfx950 (REST article, section "REST: 基于检索的投机解码"):
// the retrieved candidate continuations form a trie whose node weights count the candidates
// carrying each prefix; the draft is the subtree of the highest-weight nodes, laid out by
// breadth-first traversal (the pseudo-sequence) with a tree-attention mask that lets each
// token see only its own ancestors.
//
// One 256-thread workgroup per sequence, everything in LDS (70 KB).  No trie is materialised:
// a node is identified by (c, d), the lowest-indexed candidate c that carries the prefix, and
// the prefix length d.  With lcp(c, c') the common-prefix length of two candidates,
//   (c, d) is a node            iff  d <= len(c) and lcp(c, c') < d for every c' < c,
//   its weight                  =    #{c' : lcp(c, c') >= d},
//   its parent (d >= 2)         =    (c, d-1) if that is a node, else (c*, d-1) with
//                                    c* = min{c' < c : lcp(c, c') >= d-1}.
// Nodes are ranked by the key (weight desc, depth asc, first candidate asc) -- a parent always
// ranks before its children, so the first N-1 form a subtree -- and the breadth-first index of
// a kept node is 1 + (#kept nodes of smaller depth) + (#kept nodes of its depth whose path of
// sibling ranks is lexicographically smaller), siblings ranked by the same key.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr int kRestThreads = 256;
constexpr int kRestKeyWords = 1 + (kRestMaxL - 7 + 7) / 8;  // depth + up to kRestMaxL levels

constexpr int kLcpStride = kRestMaxM + 4;  // bytes per lcp row: rows 33 words apart, so the
                                           // rows read by one wave fall in different banks

struct RestLds {
  int32_t cand[kRestMaxL * kRestMaxM];        // token t of candidate c at t * kRestMaxM + c
  uint8_t lcp[kRestMaxM * kLcpStride];        // common-prefix lengths of candidate pairs
  uint32_t key[kRestMaxM * kRestMaxL];        // node keys (compacted); sorted if many
  uint32_t sel[kRestMaxN];                    // kept node keys in rank order
  uint8_t first[kRestMaxM * kRestMaxL];       // min{c' < c : lcp(c, c') >= d}, 0xFF if none
  int16_t sel_of[kRestMaxM * kRestMaxL];      // kept index of node (c, d) (slot c * L + d - 1)
  uint64_t bkey[kRestMaxN][kRestKeyWords];    // breadth-first keys
  uint8_t anc[kRestMaxN][kRestMaxL + 1];      // BFS indices of the ancestors by depth
  uint8_t depth_of[kRestMaxN];                // depth by BFS index
  int16_t par[kRestMaxN];                     // kept index of the parent (-1: the root)
  int16_t bfs[kRestMaxN];                     // breadth-first index of kept node s
  uint8_t sr[kRestMaxN];                      // rank among siblings
  uint8_t len[kRestMaxM];
  int nnodes, nroot;
};

__device__ __forceinline__ uint32_t rest_key(int w, int d, int c) {
  return ((uint32_t)(255 - w) << 13) | ((uint32_t)d << 7) | (uint32_t)c;
}

__global__ __launch_bounds__(kRestThreads) void k_rest_tree(
    const int32_t* __restrict__ cands, int M, int L, int N, int32_t* __restrict__ out_parent,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_n, int32_t* __restrict__ out_depth,
    int32_t* __restrict__ out_weight, uint8_t* __restrict__ out_mask) {
  __shared__ RestLds S;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int ML = M * L;
  const int32_t* src = cands + (size_t)b * ML;
  // transpose into LDS: consecutive threads take consecutive candidates of one position
  for (int i = tid; i < ML; i += kRestThreads) {
    const int t = i / M, c = i - t * M;
    S.cand[t * kRestMaxM + c] = src[(size_t)c * L + t];
  }
  if (tid == 0) {
    S.nnodes = 0;
    S.nroot = 0;
  }
  __syncthreads();

  // lengths (a candidate ends at its first negative entry)
  for (int c = tid; c < M; c += kRestThreads) {
    int l = 0;
    while (l < L && S.cand[l * kRestMaxM + c] >= 0) ++l;
    S.len[c] = (uint8_t)l;
    if (l > 0) atomicAdd(&S.nroot, 1);
  }
  __syncthreads();

  // common-prefix length of every ordered pair: a pass covers 256 / M rows c, consecutive
  // threads taking consecutive c2; all tokens are compared (independent loads)
  {
    const int rpp = kRestThreads / M;
    const int r = tid / M, c2 = tid - r * M;
    if (r < rpp) {
      for (int c = r; c < M; c += rpp) {
        const int lim = S.len[c] < S.len[c2] ? S.len[c] : S.len[c2];
        int l = 0, alive = 1;
#pragma unroll 8
        for (int t = 0; t < L; ++t) {
          alive &= (t < lim) & (S.cand[t * kRestMaxM + c] == S.cand[t * kRestMaxM + c2]);
          l += alive;
        }
        S.lcp[c * kLcpStride + c2] = (uint8_t)l;
      }
    }
  }
  __syncthreads();

  // per slot (c, d): weight = #{c2 : lcp >= d}, first = min{c2 < c : lcp >= d}; (c, d) is a
  // node iff d <= len(c) and no earlier candidate carries the prefix; node keys are appended
  // to S.key (order of arrival: only their ranks are used)
  for (int i0 = 0; i0 < ML; i0 += kRestThreads) {  // uniform trip count: the ballot below
    const int i = i0 + tid;
    const int c = i / L, d = i - c * L + 1;
    bool node = false;
    uint32_t key = 0u;
    if (i < ML) {
      // bytewise over 4 pairs a word (lcp <= 32 < 128, d <= 32): the top bit of each byte of
      // (x | 0x80808080) - d * 0x01010101 is set iff that byte is >= d, with no borrow
      // between bytes
      const uint32_t dd = (uint32_t)d * 0x01010101u;
      const uint32_t* row = reinterpret_cast<const uint32_t*>(S.lcp + c * kLcpStride);
      const int nwords = (M + 3) >> 2;
      int w = 0, fst = 0xFF;
#pragma unroll 4
      for (int wi = 0; wi < nwords; ++wi) {
        const int c0 = wi * 4;
        uint32_t t = ((row[wi] | 0x80808080u) - dd) & 0x80808080u;
        const int valid = M - c0 < 4 ? M - c0 : 4;  // candidates in this word
        t &= valid >= 4 ? 0xFFFFFFFFu : ((1u << (8 * valid)) - 1u);
        w += __popc(t);
        const int before = c - c0;  // bytes of candidates below c
        const uint32_t tb = before >= 4 ? t : (before <= 0 ? 0u : t & ((1u << (8 * before)) - 1u));
        const int hit = tb ? c0 + ((__ffs(tb) - 1) >> 3) : 0xFF;
        fst = hit < fst ? hit : fst;
      }
      S.first[i] = (uint8_t)fst;
      node = d <= S.len[c] && fst == 0xFF;
      key = rest_key(w, d, c);
    }
    // one LDS atomic per wave reserves the wave's slots
    const unsigned long long nm = __ballot(node);
    int base = 0;
    if ((threadIdx.x & 63) == 0 && nm) base = atomicAdd(&S.nnodes, __popcll(nm));
    base = __shfl(base, 0);
    if (node) S.key[base + __popcll(nm & ((1ull << (threadIdx.x & 63)) - 1ull))] = key;
  }
  __syncthreads();

  // ranks of the node keys (all distinct): by counting when there are few, else a bitonic
  // sort of the compacted keys
  const int nn = S.nnodes;
  const int nsel = min(N - 1, nn);
  if (nn <= 2 * kRestThreads) {
    if (tid < 4) S.key[nn + tid] = 0xFFFFFFFFu;  // pad to whole 4-key vectors
    __syncthreads();
    const uint4* kv = reinterpret_cast<const uint4*>(S.key);
    for (int j = tid; j < nn; j += kRestThreads) {
      const uint32_t kj = S.key[j];
      int rank = 0;
#pragma unroll 4
      for (int k4 = 0; k4 < ((nn + 3) >> 2); ++k4) {
        const uint4 x = kv[k4];
        rank += (x.x < kj) + (x.y < kj) + (x.z < kj) + (x.w < kj);
      }
      if (rank < nsel) S.sel[rank] = kj;
    }
  } else {
    int SP = 2;
    while (SP < nn) SP <<= 1;
    for (int i = nn + tid; i < SP; i += kRestThreads) S.key[i] = 0xFFFFFFFFu;
    for (int size = 2; size <= SP; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        __syncthreads();
        for (int t = tid; t < (SP >> 1); t += kRestThreads) {
          const int i = ((t & ~(stride - 1)) << 1) | (t & (stride - 1));
          const int l = i + stride;
          const uint32_t a = S.key[i], c = S.key[l];
          const bool up = (i & size) == 0;
          if (up ? a > c : a < c) {
            S.key[i] = c;
            S.key[l] = a;
          }
        }
      }
    __syncthreads();
    for (int r = tid; r < nsel; r += kRestThreads) S.sel[r] = S.key[r];
  }
  __syncthreads();

  // decode the kept nodes, then their parents
  int my_c = 0, my_d = 0, my_w = 0;
  if (tid < nsel) {
    const uint32_t k = S.sel[tid];
    my_c = (int)(k & 127u);
    my_d = (int)((k >> 7) & 63u);
    my_w = 255 - (int)(k >> 13);
    S.sel_of[my_c * L + my_d - 1] = (int16_t)tid;
  }
  __syncthreads();
  if (tid < nsel) {
    int p = -1;
    if (my_d >= 2) {
      const int f = S.first[my_c * L + my_d - 2];  // first earlier carrier of the parent
      const int cp = f == 0xFF ? my_c : f;
      p = cp < M ? S.sel_of[cp * L + my_d - 2] : -1;
    }
    S.par[tid] = (int16_t)p;
  }
  __syncthreads();
  // sibling ranks: kept nodes are in key order, which orders siblings as required
  if (tid < nsel) {
    const int p = S.par[tid];
    int r = 0;
#pragma unroll 8
    for (int s = 0; s < tid; ++s) r += S.par[s] == p;  // siblings: the same parent
    S.sr[tid] = (uint8_t)r;
  }
  __syncthreads();
  // breadth-first key: (depth, sibling ranks from the top) compared lexicographically, packed
  // in 64-bit words, most significant first -- word 0 holds the depth and levels 0..6, each
  // further word 8 levels
  if (tid < nsel) {
    uint64_t* kw = S.bkey[tid];
    for (int w = 0; w < kRestKeyWords; ++w) kw[w] = 0ull;
    kw[0] = (uint64_t)my_d << 56;
    uint8_t* kb = reinterpret_cast<uint8_t*>(kw);
    int a = tid;
    for (int lvl = my_d - 1; lvl >= 0; --lvl) {
      const int w = lvl < 7 ? 0 : 1 + (lvl - 7) / 8;
      const int byte = lvl < 7 ? 6 - lvl : 7 - (lvl - 7) % 8;  // within the little-endian word
      kb[w * 8 + byte] = S.sr[a];
      a = S.par[a];
    }
  }
  __syncthreads();
  // breadth-first index = 1 + #{kept nodes with a smaller key}: word 0 first; nodes equal in
  // it (same depth below 8, same first 7 levels) compare their further words
  if (tid < nsel) {
    const uint64_t k0 = S.bkey[tid][0];
    const int nw = my_d <= 7 ? 1 : 1 + (my_d - 7 + 7) / 8;
    int idx = 1, ties = 0;
#pragma unroll 8
    for (int s = 0; s < nsel; ++s) {
      const uint64_t x = S.bkey[s][0];
      idx += x < k0;
      ties += x == k0;
    }
    if (ties > 1) {
      for (int s = 0; s < nsel; ++s) {
        if (s == tid || S.bkey[s][0] != k0) continue;
        int cmp = 0;
        for (int w = 1; w < nw && cmp == 0; ++w) {
          const uint64_t y = S.bkey[s][w], z = S.bkey[tid][w];
          cmp = y < z ? -1 : (y > z ? 1 : 0);
        }
        idx += cmp < 0;
      }
    }
    S.bfs[tid] = (int16_t)idx;
  }
  __syncthreads();

  // outputs in breadth-first order; ancestor table (BFS indices by depth) for the mask
  const int n = 1 + nsel;
  int32_t* o_par = out_parent + (size_t)b * N;
  int32_t* o_tok = out_tokens + (size_t)b * N;
  if (tid < nsel) {
    const int i = S.bfs[tid];
    const int p = S.par[tid];
    o_par[i] = p < 0 ? 0 : S.bfs[p];
    o_tok[i] = S.cand[(my_d - 1) * kRestMaxM + my_c];
    if (out_depth) out_depth[(size_t)b * N + i] = my_d;
    if (out_weight) out_weight[(size_t)b * N + i] = my_w;
    S.anc[i][0] = 0;
    int a = tid;
    for (int lvl = my_d; lvl >= 1; --lvl) {
      S.anc[i][lvl] = (uint8_t)S.bfs[a];
      a = S.par[a];
    }
    S.depth_of[i] = (uint8_t)my_d;
  }
  if (tid == 0) {
    o_par[0] = -1;
    o_tok[0] = -1;
    if (out_depth) out_depth[(size_t)b * N] = 0;
    if (out_weight) out_weight[(size_t)b * N] = S.nroot;
    S.anc[0][0] = 0;
    S.depth_of[0] = 0;
    out_n[b] = n;
  }
  for (int i = n + tid; i < N; i += kRestThreads) {
    o_par[i] = -1;
    o_tok[i] = -1;
    if (out_depth) out_depth[(size_t)b * N + i] = -1;
    if (out_weight) out_weight[(size_t)b * N + i] = -1;
  }
  if (out_mask) {
    __syncthreads();
    // thread = one column j over rows i0, i0 + step, ...: node j is in row i's set iff it is
    // node i's ancestor at its own depth
    uint8_t* mrow = out_mask + (size_t)b * N * N;
    const int step = kRestThreads / N;
    const int i0 = tid / N, j = tid - i0 * N;
    if (i0 < step) {
      const int dj = j < n ? S.depth_of[j] : 0;
#pragma unroll 4
      for (int i = i0; i < N; i += step) {
        uint8_t v = 0;
        if (i < n && j < n) v = (dj <= S.depth_of[i] && S.anc[i][dj] == j) ? 1 : 0;
        mrow[(size_t)i * N + j] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_rest_tree(const int32_t* cands, int B, int M, int L, int N, int32_t* parent,
                            int32_t* tokens, int32_t* n_nodes, int32_t* depth, int32_t* weight,
                            uint8_t* mask, hipStream_t stream) {
  hipLaunchKernelGGL(k_rest_tree, dim3(B), dim3(kRestThreads), 0, stream, cands, M, L, N, parent,
                     tokens, n_nodes, depth, weight, mask);
  return hipGetLastError();
}

}  // namespace sv
