// HIP kernels for gfx950 (CDNA4): verify-and-resample of speculative sampling and greedy tree
// verification.  Every row of logits is streamed from HBM once by k_chunk with coalesced
// 16-byte loads and kept in registers while it is reduced; all later kernels touch only small
// per-row summaries, except where a row has no compact summary (no truncation, top-p, or a
// top-k tie set too large for the candidate lists), where the final draw re-reads one row pair.
//
// Method (page "Accelerating Large Language Model Decoding with Speculative Sampling", Chen et
// al. notes; q = target, p = draft): section A2 "modified rejection sampling" for the accept
// test and the (q - p)_+ residual, the bonus-token remark of the same section, Theorem 1 in the
// appendix; temperature / top-k / top-p applied before the scheme (section A2, compatibility
// with standard sampling methods); lenience from App. F of the "Fast Inference from
// Transformers via Speculative Decoding" blog; greedy tree acceptance from the REST article.
//
// Reductions use fixed orders only (wave butterflies, then the 4 waves in order; chunks in
// order; kept tokens in index order), and integer atomics only, so results are bitwise
// reproducible.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

#include "sv_internal.hpp"

namespace sv {
namespace {

// ------------------------------------------------------------------------------------------
// Element traits.  bf16 is handled as raw 16-bit patterns, two per 32-bit register.
//
// Keys: an order-preserving map from the element's bits to an unsigned integer (flip all bits
// of negatives, set the sign bit of non-negatives).  -0 and +0 get adjacent keys; canon()
// merges them, so that equal floating-point values have equal keys.
// ------------------------------------------------------------------------------------------
template <class E>
struct Tr;

template <>
struct Tr<uint16_t> {
  static constexpr int kEpv = 8;        // elements per 16-byte vector
  static constexpr int kPerDword = 2;   // elements per 32-bit register
  static constexpr int kKeyBits = 16;
  static constexpr uint32_t kKeyPos0 = 0x8000u;
  static constexpr uint32_t kKeyNeg0 = 0x7FFFu;
  static constexpr uint32_t kNegInfPair = 0xFF80FF80u;  // two -inf

  __device__ static float elem(uint32_t w, int h) {
    return __uint_as_float(h ? (w & 0xFFFF0000u) : (w << 16));
  }
  __device__ static uint32_t bits_of(uint16_t v) { return v; }
  __device__ static float to_float(uint32_t bits) { return __uint_as_float(bits << 16); }
  __device__ static uint32_t key_of_bits(uint32_t b) {
    return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
  }
  // two keys at once: per 16-bit half, bits ^ (negative ? 0xFFFF : 0x8000)
  __device__ static uint32_t keys_of_dword(uint32_t w) {
    typedef short s2 __attribute__((ext_vector_type(2)));
    s2 v = __builtin_bit_cast(s2, w);
    s2 sh = v >> (s2){15, 15};
    return w ^ (__builtin_bit_cast(uint32_t, sh) | 0x80008000u);
  }
  __device__ static uint32_t dword_max(uint32_t a, uint32_t b) {
    typedef unsigned short u2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(
        uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u2, a), __builtin_bit_cast(u2, b)));
  }
  __device__ static uint32_t dword_hmax(uint32_t w) {
    uint32_t lo = w & 0xFFFFu, hi = w >> 16;
    return lo > hi ? lo : hi;
  }
  __device__ static float key_to_float(uint32_t key) {
    uint32_t b = (key & 0x8000u) ? (key ^ 0x8000u) : (~key & 0xFFFFu);
    return __uint_as_float(b << 16);
  }
  __device__ static uint32_t canon(uint32_t key) { return key == kKeyNeg0 ? kKeyPos0 : key; }
};

template <>
struct Tr<float> {
  static constexpr int kEpv = 4;
  static constexpr int kPerDword = 1;
  static constexpr int kKeyBits = 32;
  static constexpr uint32_t kKeyPos0 = 0x80000000u;
  static constexpr uint32_t kKeyNeg0 = 0x7FFFFFFFu;
  static constexpr uint32_t kNegInfPair = 0xFF800000u;

  __device__ static float elem(uint32_t w, int) { return __uint_as_float(w); }
  __device__ static uint32_t bits_of(float v) { return __float_as_uint(v); }
  __device__ static float to_float(uint32_t bits) { return __uint_as_float(bits); }
  __device__ static uint32_t key_of_bits(uint32_t b) {
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  __device__ static uint32_t keys_of_dword(uint32_t w) {
    return w ^ ((uint32_t)((int32_t)w >> 31) | 0x80000000u);
  }
  __device__ static uint32_t dword_max(uint32_t a, uint32_t b) { return a > b ? a : b; }
  __device__ static uint32_t dword_hmax(uint32_t w) { return w; }
  __device__ static float key_to_float(uint32_t key) {
    uint32_t b = (key & 0x80000000u) ? (key ^ 0x80000000u) : ~key;
    return __uint_as_float(b);
  }
  __device__ static uint32_t canon(uint32_t key) { return key == kKeyNeg0 ? kKeyPos0 : key; }
};

// e^x in fp32 for x <= 0 (every weight here is exp((z - m) / T) with z <= m): the hardware
// base-2 exponential of x * log2(e).  Every fp32 weight in the library goes through this one
// function, so the normalisers and the weights they normalise agree.
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

constexpr int kRegs = kVecPerThread * 4;  // 32-bit registers per thread holding one chunk

// One logit of a row, as a float.
template <class E>
__device__ __forceinline__ float load_logit(const E* row, int idx) {
  return Tr<E>::to_float(Tr<E>::bits_of(row[idx]));
}

// ------------------------------------------------------------------------------------------
// Block reductions (256 threads = 4 waves of 64).  Fixed butterfly inside a wave, then the
// four wave results in order: deterministic.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
// Lanes of the wave below this one, as a ballot mask.
__device__ __forceinline__ unsigned long long lanes_below() {
  return (1ull << lane_id()) - 1ull;
}

// base + the number of set bits of mask in the lanes below this one (two mbcnt instructions).
__device__ __forceinline__ int lane_rank(unsigned long long mask, int base) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, (uint32_t)base));
}

// 2 mk + (x < n), unsigned: the borrow of x - n (left in VCC by v_sub_co_u32) is the carry-in
// of mk + mk (v_addc_co_u32), with the two wait states a VALU read of a VALU-written VCC needs.
__device__ __forceinline__ uint32_t shift_in_lt(uint32_t mk, uint32_t x, uint32_t n) {
  uint32_t out, diff;
  asm("v_sub_co_u32 %1, vcc, %2, %3\n\ts_nop 1\n\tv_addc_co_u32 %0, vcc, %4, %4, vcc"
      : "=v"(out), "=&v"(diff)
      : "v"(x), "v"(n), "v"(mk)
      : "vcc");
  return out;
}

// The value of lane (this lane ^ O), with no lane-address register: below 32 a ds_swizzle in
// bit-mask mode (and 0x1F, xor O: an immediate pattern); across the halves v_permlane32_swap,
// which exchanges the upper half of its first operand with the lower half of its second (both
// v here), so the lower lanes find their partner in the second result, the upper lanes in the
// first.
template <int O>
__device__ __forceinline__ int xor_lane_i(int v) {
  if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return lane_id() < 32 ? (int)r[1] : (int)r[0];
  } else {
    return __builtin_amdgcn_ds_swizzle(v, 0x1F | (O << 10));
  }
}
template <int O, class T>
__device__ __forceinline__ T xor_lane(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, xor_lane_i<O>(__builtin_bit_cast(int, v)));
  } else {
    typedef int i2 __attribute__((ext_vector_type(2)));
    i2 x = __builtin_bit_cast(i2, v);
    x.x = xor_lane_i<O>(x.x);
    x.y = xor_lane_i<O>(x.y);
    return __builtin_bit_cast(T, x);
  }
}

template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, xor_lane<32>(v));
  v = op(v, xor_lane<16>(v));
  v = op(v, xor_lane<8>(v));
  v = op(v, xor_lane<4>(v));
  v = op(v, xor_lane<2>(v));
  v = op(v, xor_lane<1>(v));
  return v;
}

// N values per lane (N a power of two, at most 64) reduced across the wave by recursive
// halving: at the exchange with lane ^ O a lane keeps the upper half of its live values if bit
// O of its lane id is set, else the lower half, and combines them with the partner's copies of
// the same values, so each step halves the live values: N - 1 combines, then 6 - log2 N
// butterfly steps on the one value left, against 6 N combines for N separate butterflies.
// Returns the total of value (lane >> (6 - log2 N)); the lanes that share those bits all
// hold it.
template <int O, int C, int N, class T, class Op>
__device__ __forceinline__ void halving_step(T (&v)[N], Op op) {  // C of the N values live
  const bool up = (lane_id() & O) != 0;
#pragma unroll
  for (int j = 0; j < C / 2; ++j) {
    const T keep = up ? v[j + C / 2] : v[j];
    const T send = up ? v[j] : v[j + C / 2];
    v[j] = op(keep, xor_lane<O>(send));
  }
}
constexpr int log2_pow2(int n) { return n <= 1 ? 0 : 1 + log2_pow2(n / 2); }

template <int N, class T, class Op>
__device__ __forceinline__ T wave_reduce_halving(T (&v)[N], Op op) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "a power of two up to 64");
  if constexpr (N >= 2) halving_step<32, N>(v, op);
  if constexpr (N >= 4) halving_step<16, N / 2>(v, op);
  if constexpr (N >= 8) halving_step<8, N / 4>(v, op);
  if constexpr (N >= 16) halving_step<4, N / 8>(v, op);
  if constexpr (N >= 32) halving_step<2, N / 16>(v, op);
  if constexpr (N >= 64) halving_step<1, N / 32>(v, op);
  // the value left in v[0] is this lane's share of value lane >> (6 - log2 N); the lanes that
  // share those bits add their shares
  T t = v[0];
  if constexpr (N < 64) t = op(t, xor_lane<1>(t));
  if constexpr (N < 32) t = op(t, xor_lane<2>(t));
  if constexpr (N < 16) t = op(t, xor_lane<4>(t));
  if constexpr (N < 8) t = op(t, xor_lane<8>(t));
  if constexpr (N < 4) t = op(t, xor_lane<16>(t));
  if constexpr (N < 2) t = op(t, xor_lane<32>(t));
  return t;
}

struct RedScratch {
  double d[4];
  float f[4];
  int i[4];
  unsigned long long u[4];
};

__device__ double block_sum_d(double v, RedScratch& s) {
  v = wave_reduce(v, [](double a, double b) { return a + b; });
  __syncthreads();
  if (lane_id() == 0) s.d[wave_id()] = v;
  __syncthreads();
  return ((s.d[0] + s.d[1]) + s.d[2]) + s.d[3];
}

__device__ float block_max_f(float v, RedScratch& s) {
  v = wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
  __syncthreads();
  if (lane_id() == 0) s.f[wave_id()] = v;
  __syncthreads();
  return fmaxf(fmaxf(s.f[0], s.f[1]), fmaxf(s.f[2], s.f[3]));
}

__device__ int block_min_i(int v, RedScratch& s) {
  v = wave_reduce(v, [](int a, int b) { return a < b ? a : b; });
  __syncthreads();
  if (lane_id() == 0) s.i[wave_id()] = v;
  __syncthreads();
  int a = s.i[0] < s.i[1] ? s.i[0] : s.i[1];
  int b = s.i[2] < s.i[3] ? s.i[2] : s.i[3];
  return a < b ? a : b;
}

__device__ int block_max_i(int v, RedScratch& s) {
  v = wave_reduce(v, [](int a, int b) { return a > b ? a : b; });
  __syncthreads();
  if (lane_id() == 0) s.i[wave_id()] = v;
  __syncthreads();
  int a = s.i[0] > s.i[1] ? s.i[0] : s.i[1];
  int b = s.i[2] > s.i[3] ? s.i[2] : s.i[3];
  return a > b ? a : b;
}

// ------------------------------------------------------------------------------------------
// Row addressing.  With rows_per_seq == 2K+1 a sequence's rows are ordered
// target 0..K, then draft 0..K-1; with rows_per_seq == 1 rows are consecutive in `t`.
// ------------------------------------------------------------------------------------------
template <class E>
__device__ __forceinline__ const E* row_ptr(const Dims& dm, const E* t, const E* d, int r) {
  if (dm.rows_per_seq == 1) return t + (size_t)r * dm.V;
  const int b = r / dm.rows_per_seq;
  const int j = r - b * dm.rows_per_seq;
  if (j <= dm.K) return t + ((size_t)b * (dm.K + 1) + j) * dm.V;
  return d + ((size_t)b * dm.draft_rows + (j - dm.K - 1)) * dm.V;
}

__device__ __forceinline__ int target_row(const Dims& dm, int b, int k) {
  return b * dm.rows_per_seq + k;
}
__device__ __forceinline__ int draft_row(const Dims& dm, int b, int k) {
  return b * dm.rows_per_seq + dm.K + 1 + k;
}

// Work item of workgroup b out of n.  Workgroups go to the eight XCDs round-robin (workgroup b
// to XCD b mod 8); this gives each XCD one contiguous range of items, taken in order, instead
// of every eighth item (measured: 1-2% less time for k_topk_row and k_topp_cand, but 3% more
// for k_chunk, which keeps the plain order).  Items past the last
// multiple of 8 keep their index, so the map is a bijection on [0, n).
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
  const int q = n >> 3;
  if (b >= (q << 3)) return b;
  return (b & 7) * q + (b >> 3);
}

// Elements of a row before its first 16-byte boundary (the row's 16-byte phase).
template <class E>
__device__ __forceinline__ int row_phase(const E* row) {
  return (int)(((uint32_t)reinterpret_cast<uintptr_t>(row) & 15u) / sizeof(E));
}

// Load this thread's share of chunk c of a row, the chunks counted from the 16-byte boundary at
// or before the row start (the row's frame: frame index a holds element a - ph, ph = the row's
// phase), so that every load is an aligned 16-byte vector: vector i of thread t covers frame
// indices c*CH + (t + 256 i) * EPV .. + EPV - 1.  The loads are range-checked raw buffer loads
// over the chunk's part of the frame, rounded up to whole vectors: the first and last vector of a
// row may take a few bytes of the neighbouring rows (the same 16-byte blocks, never another
// page); those slots, and slots past the row end, get `fill`.  Returns ph: the element index of
// slot_index(c0, ...) is then slot_index(c * CH - ph, ...).
// NV vectors per thread over frame indices [c0, c0 + ce) (a whole chunk, or a part of one).
template <class E, int NV = kVecPerThread>
__device__ __forceinline__ int load_frame_part(const E* __restrict__ row, int V, int c0, int ce,
                                               uint32_t (&regs)[4 * NV], uint32_t fill) {
  constexpr int EPV = Tr<E>::kEpv;
  const int tid = threadIdx.x;
  const int ph = row_phase(row);
  const int fl = V + ph;  // frame length
  const int flen = max(0, min(ce, fl - c0));
  const int bytes = min(ce * (int)sizeof(E), (flen * (int)sizeof(E) + 15) & ~15);
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  // Logits are read exactly once, so the loads are non-temporal (cache policy bit 1).
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<E*>(row - ph + c0), (short)0, bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, i * kThreads * 16, 2);
    regs[4 * i + 0] = x.x;
    regs[4 * i + 1] = x.y;
    regs[4 * i + 2] = x.z;
    regs[4 * i + 3] = x.w;
  }
  // slots outside [ph, fl): whole vectors past the end, and the row's first and last vector
  // (only chunks holding the row's start or end have any)
  if (c0 >= ph && c0 + ce <= fl) return ph;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int a0 = c0 + (tid + kThreads * i) * EPV;
    if (a0 >= ph && a0 + EPV <= fl) continue;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t w = regs[4 * i + d];
#pragma unroll
      for (int h = 0; h < Tr<E>::kPerDword; ++h) {
        const int a = a0 + d * Tr<E>::kPerDword + h;
        if (a < ph || a >= fl) {
          if constexpr (Tr<E>::kPerDword == 2) {
            const uint32_t m = 0xFFFFu << (16 * h);
            w = (w & ~m) | (fill & m);
          } else {
            w = fill;
          }
        }
      }
      regs[4 * i + d] = w;
    }
  }
  return ph;
}

template <class E>
__device__ __forceinline__ int load_chunk_frame(const E* __restrict__ row, int V, int c, int ce,
                                                uint32_t (&regs)[kRegs], uint32_t fill) {
  return load_frame_part<E>(row, V, c * ce, ce, regs, fill);
}

// Element index of slot (vector i, register d, half h) of this thread in chunk starting at c0.
template <class E>
__device__ __forceinline__ int slot_index(int c0, int i, int d, int h) {
  return c0 + (threadIdx.x + kThreads * i) * Tr<E>::kEpv + d * Tr<E>::kPerDword + h;
}

// ------------------------------------------------------------------------------------------
// k_chunk: one workgroup per (row, chunk).  Reads each logit of the chunk once: vmax and
// sum exp((z - vmax) / T) over the chunk (HIST: and the chunk's top-p mass histogram).
// ROWSTAT: a row of one chunk with nothing truncated, whose row statistics are the chunk's
// own; they are written here and the merge over chunks is not launched.
// ------------------------------------------------------------------------------------------
// Grid edge of a logit for the top-p mass histogram: floor(8 z / T), clamped so that any finite
// logit (and -inf) maps to an int.  Every kernel bins with this one function.
__device__ __forceinline__ int topp_edge(float z, float it) {
  float f = floorf(z * it * (float)kHistPerUnit);
  f = fminf(fmaxf(f, -1073741824.0f), 1073741824.0f);
  return (int)f;
}

template <class E, bool HIST = false, bool ROWSTAT = false>
__global__ __launch_bounds__(kThreads) void k_chunk(const E* __restrict__ tgt,
                                                    const E* __restrict__ drf, Dims dm, Samp sp,
                                                    Workspace ws) {
  const int bid = blockIdx.x;  // (the XCD-contiguous order measured slower here)
  const int r = bid / dm.nchunks;
  const int c = bid - r * dm.nchunks;
  const E* row = row_ptr(dm, tgt, drf, r);
  const int tid = threadIdx.x;
  __shared__ RedScratch red;

  uint32_t regs[kRegs];
  ChunkPart* part = ws.parts + (size_t)r * dm.nchunks + c;

  constexpr int NBINS = sizeof(E) == 4 ? kHistBinsF32 : kHistBins;
  __shared__ unsigned long long s_hist[HIST ? NBINS : 1];
  if constexpr (HIST)
    for (int j = tid; j < NBINS; j += kThreads) s_hist[j] = 0ull;
  // element index of the chunk's first slot (negative for a row's first chunk when unaligned)
  const int c0 = c * dm.chunk_elems -
                 load_chunk_frame<E>(row, dm.V, c, dm.chunk_elems, regs, Tr<E>::kNegInfPair);
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kRegs; ++j) {
#pragma unroll
    for (int h = 0; h < Tr<E>::kPerDword; ++h) mx = fmaxf(mx, Tr<E>::elem(regs[j], h));
  }
  mx = block_max_f(mx, red);
  // Opaque to the compiler, so that the second pass decodes the elements again instead of
  // keeping every decoded value live across the reduction.
#pragma unroll
  for (int j = 0; j < kRegs; ++j) asm volatile("" : "+v"(regs[j]));
  ChunkPart p;
  p.vmax = mx;
  p.argmax = -1;
  p.sum = 0.0;
  p.pad[0] = p.pad[1] = p.pad[2] = p.pad[3] = 0;
  {
    double s = 0.0;
    const float it = sp.inv_t;
    const int etop = topp_edge(mx, it);
    // fp32 top-p rows: each element's edge code, one byte per slot of the chunk frame (byte a of
    // the chunk's codes is frame slot c * CH + a), four per vector, stored as one dword
    constexpr bool CODES = HIST && sizeof(E) == 4;
    uint32_t* codes = nullptr;
    if constexpr (CODES) codes = reinterpret_cast<uint32_t*>(
        ws.codes + ((size_t)r * dm.nchunks + c) * dm.chunk_elems);
    if (mx > -INFINITY) {
#pragma unroll
      for (int i = 0; i < kVecPerThread; ++i) {
        float sv = 0.f;  // one vector's EPV terms in fp32, then into the fp64 total
        uint32_t cw = 0u;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int h = 0; h < Tr<E>::kPerDword; ++h) {
            const float z = Tr<E>::elem(regs[4 * i + d], h);
            const float e = fast_exp((z - mx) * it);
            sv += e;
            if constexpr (HIST) {
              // mass in 2^-40 fixed point relative to the chunk maximum, so that the bin sums
              // are exact integer additions whatever their order
              uint32_t code = kCodeFar;
              if (e > 0.0f) {
                const int g = etop - topp_edge(z, it);
                const int j = min(g, NBINS - 1);
                atomicAdd(&s_hist[j], __float2ull_rz(e * 1099511627776.0f));
                code = (uint32_t)min(g, kCodeFar);
              }
              cw |= code << (8 * d);
            }
          }
        }
        if constexpr (CODES) codes[threadIdx.x + kThreads * i] = cw;
        s += (double)sv;
      }
    } else if constexpr (CODES) {
#pragma unroll
      for (int i = 0; i < kVecPerThread; ++i) codes[threadIdx.x + kThreads * i] = 0xFFFFFFFFu;
    }
    p.sum = block_sum_d(s, red);  // its barriers also order the histogram updates
    if constexpr (HIST) {
      unsigned long long* dst = ws.hist + ((size_t)r * dm.nchunks + c) * NBINS;
      for (int j = tid; j < NBINS; j += kThreads) dst[j] = s_hist[j];
      p.pad[0] = etop;
    }
  }
  if (tid == 0) {
    *part = p;
    if constexpr (ROWSTAT) {  // the row is this one chunk and nothing is truncated
      RowStat out;
      out.m = mx;
      out.thr = -INFINITY;
      out.S = p.sum;
      out.argmax = -1;
      out.nkept = -1;
      out.kind = kRowDense;
      out.pad = 0;
      ws.rstat[r] = out;
    }
  }
}

// Argmax of one (row, chunk): the chunk's maximum and the lowest index holding it, in one pass
// over two half-tiles (32 registers per thread, so that more workgroups are resident than with
// the dense path's whole-tile registers).  A thread visits its slots in increasing index
// order, so a strict comparison keeps the lowest index of its maximum; slots outside the row
// hold -inf.  Writes the same ChunkPart as k_chunk's argmax mode.
template <class E>
__global__ __launch_bounds__(kThreads) void k_chunk_argmax(const E* __restrict__ tgt,
                                                           const E* __restrict__ drf, Dims dm,
                                                           Samp sp, Workspace ws) {
  constexpr int NV = kVecPerThread / 2;
  const int r = blockIdx.x / dm.nchunks;
  const int c = blockIdx.x - r * dm.nchunks;
  const E* row = row_ptr(dm, tgt, drf, r);
  const int half = dm.chunk_elems / 2;
  __shared__ RedScratch red;
  float bv = -INFINITY;
  int bi = INT_MAX;
#pragma unroll 1
  for (int part = 0; part < 2; ++part) {
    uint32_t regs[4 * NV];
    const int f0 = c * dm.chunk_elems + part * half;  // frame index of the part's start
    const int e0 = f0 - load_frame_part<E, NV>(row, dm.V, f0, half, regs, Tr<E>::kNegInfPair);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int h = 0; h < Tr<E>::kPerDword; ++h) {
          const float z = Tr<E>::elem(regs[4 * i + d], h);
          if (z > bv) {
            bv = z;
            bi = slot_index<E>(e0, i, d, h);
          }
        }
      }
    }
  }
  const float mx = block_max_f(bv, red);
  int best = block_min_i(bv == mx && mx > -INFINITY ? bi : INT_MAX, red);
  if (!(mx > -INFINITY)) best = max(c * dm.chunk_elems - row_phase(row), 0);
  (void)sp;
  if (threadIdx.x == 0) {
    ChunkPart p;
    p.vmax = mx;
    p.argmax = best;
    p.sum = 0.0;
    p.pad[0] = p.pad[1] = p.pad[2] = p.pad[3] = 0;
    ws.parts[(size_t)r * dm.nchunks + c] = p;
  }
}

// ------------------------------------------------------------------------------------------
// Whole-row helpers for k_row's selection paths (re-read the row from memory).
// ------------------------------------------------------------------------------------------
template <class E, bool VEC, class F>
__device__ __forceinline__ void row_foreach(const E* __restrict__ row, int V, F&& f) {
  constexpr int EPV = Tr<E>::kEpv;
  if constexpr (VEC) {
    const uint4* vp = reinterpret_cast<const uint4*>(row);
    const int nvec = V / EPV;
    for (int v = threadIdx.x; v < nvec; v += kThreads) {
      const uint4 x = vp[v];
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int h = 0; h < Tr<E>::kPerDword; ++h) {
          const uint32_t bits =
              (Tr<E>::kPerDword == 2) ? (h ? (w[d] >> 16) : (w[d] & 0xFFFFu)) : w[d];
          f(v * EPV + d * Tr<E>::kPerDword + h, Tr<E>::elem(w[d], h), bits);
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < V; i += kThreads) {
      const uint32_t bits = Tr<E>::bits_of(row[i]);
      f(i, Tr<E>::to_float(bits), bits);
    }
  }
}

template <class E, bool VEC>
__device__ double dense_sum(const E* row, int V, float m, float it, float thr, RedScratch& red) {
  double s = 0.0;
  row_foreach<E, VEC>(row, V, [&](int, float z, uint32_t) {
    if (z >= thr) s += (double)fast_exp((z - m) * it);
  });
  return block_sum_d(s, red);
}

// Largest key v with weight(key >= v) >= target, by most-significant-digit radix selection over
// canonical keys, restricted to keys >= lower.  MASS: weight = exp((z - m) / T) in 2^-40 fixed
// point (integer atomics, deterministic), target = ceil(P * total); else weight 1, target = k.
// Digits of D bits, most significant first (the last one may be narrower); s_bins holds 2^D.
// Scratch of radix_select, one copy per kernel whatever the instantiations it uses.
__shared__ unsigned long long g_radix_tot[kThreads];
__shared__ unsigned long long g_radix_target, g_radix_above;
__shared__ uint32_t g_radix_prefix;

template <class E, bool VEC, bool MASS, int D = (Tr<E>::kKeyBits == 16 ? 8 : 11)>
__device__ uint32_t radix_select(const E* row, int V, float m, float it, uint32_t lower,
                                 double P_or_k, unsigned long long* s_bins) {
  constexpr int KB = Tr<E>::kKeyBits;
  constexpr int NLEV = (KB + D - 1) / D;
  const int tid = threadIdx.x;
  unsigned long long* s_tot = g_radix_tot;
  unsigned long long& s_target = g_radix_target;
  unsigned long long& s_above = g_radix_above;
  uint32_t& s_prefix = g_radix_prefix;
  if (tid == 0) {
    s_above = 0;
    s_prefix = 0;
  }
  for (int L = 0; L < NLEV; ++L) {
    const int shift = KB - (L + 1) * D > 0 ? KB - (L + 1) * D : 0;
    const int bits = KB - L * D - shift;
    const int nb = 1 << bits;
    for (int j = tid; j < nb; j += kThreads) s_bins[j] = 0ull;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    const int hshift = shift + bits;
    row_foreach<E, VEC>(row, V, [&](int, float z, uint32_t b) {
      const uint32_t key = Tr<E>::canon(Tr<E>::key_of_bits(b));
      if (key < lower) return;
      if (L > 0 && (hshift >= 32 ? 0u : (key >> hshift)) != prefix) return;
      unsigned long long w = 1ull;
      if constexpr (MASS) w = (unsigned long long)rintf(fast_exp((z - m) * it) * 0x1p40f);
      if (w) atomicAdd(&s_bins[(key >> shift) & (uint32_t)(nb - 1)], w);
    });
    __syncthreads();
    // per-thread totals of consecutive bins, then suffix sums over threads
    const int per = nb / kThreads > 0 ? nb / kThreads : 1;
    const int b0 = tid * per;
    unsigned long long mine = 0;
    if (b0 < nb)
      for (int j = 0; j < per; ++j) mine += s_bins[b0 + j];
    s_tot[tid] = mine;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {  // inclusive suffix scan
      const unsigned long long add = (tid + off < kThreads) ? s_tot[tid + off] : 0ull;
      __syncthreads();
      s_tot[tid] += add;
      __syncthreads();
    }
    if (L == 0 && tid == 0) {
      const unsigned long long total = s_tot[0];
      unsigned long long t;
      if constexpr (MASS) {
        double tt = ceil(P_or_k * (double)total);
        t = tt < 1.0 ? 1ull : (unsigned long long)tt;
        if (t > total) t = total;
      } else {
        t = (unsigned long long)P_or_k;
      }
      s_target = t;
    }
    __syncthreads();
    const unsigned long long target = s_target;
    const unsigned long long above = s_above;
    const unsigned long long after = (tid + 1 < kThreads) ? s_tot[tid + 1] : 0ull;
    __syncthreads();
    if (b0 < nb) {
      unsigned long long cum = above + after;
      for (int j = per - 1; j >= 0; --j) {
        const unsigned long long before = cum;
        cum += s_bins[b0 + j];
        if (cum >= target && before < target) {
          s_above = before;
          s_prefix = (prefix << bits) | (uint32_t)(b0 + j);
        }
      }
    }
    __syncthreads();
  }
  return s_prefix;
}

// ------------------------------------------------------------------------------------------
// Top-p without top-k (the nucleus; Chen et al. notes, A2, and the Leviathan blog's standardised
// sampling section: the smallest set of most probable tokens whose mass reaches P).
//   k_chunk (HIST)  per chunk: a histogram of exp((z - chunk max) / T) in 2^-40 fixed point
//                   over edges floor(8 z / T), 512 edges down from the chunk maximum's (the last
//                   bin holds everything lower)
//   k_row           merges the chunk histograms onto the row maximum's edges and finds the bin
//                   where the mass, accumulated from the top, first reaches P * S; the elements
//                   of that bin and its two neighbours are the candidates, everything above is
//                   kept
//   k_topp_cand     re-reads the rows and appends the candidates to a per-row list
//   k_topp_select   sorts the candidates by logit (descending) and takes the exact boundary
// The tokens in the last bin are at least 64 units of z / T below the maximum, where the mass of
// any number of tokens that fits an int stays below 1 - P for every float P < 1, so the
// boundary is never among them unless the candidate range is already open below.
// ------------------------------------------------------------------------------------------
// Histogram loads of a batch of chunks [c0, c0 + kHistBatch) of row r (zeros past the row), so
// that callers can issue the first batch before they need it.
// NBINS bins per chunk (kHistBins for bf16 rows, kHistBinsF32 for fp32 rows).
template <int NB, int NBINS>  // chunks per batch
using HistBatch = unsigned long long[NB][NBINS / kThreads];

template <int NB, int NBINS>
__device__ __forceinline__ void hist_batch_load(const Dims& dm, const Workspace& ws, int r, int c0,
                                                int ce, HistBatch<NB, NBINS>& h) {
  // a buffer over chunks [c0, ce) of the row: loads past it read 0, with no branch
  typedef unsigned int u2 __attribute__((ext_vector_type(2)));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      ws.hist + ((size_t)r * dm.nchunks + c0) * NBINS, (short)0,
      max(0, ce - c0) * NBINS * (int)sizeof(unsigned long long), 0x00020000);
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int i = 0; i < NBINS / kThreads; ++i) {
      const u2 x = __builtin_amdgcn_raw_buffer_load_b64(
          rs, (int)((threadIdx.x + i * kThreads) * sizeof(unsigned long long)),
          q * NBINS * (int)sizeof(unsigned long long), 0);
      h[q][i] = (unsigned long long)x.x | ((unsigned long long)x.y << 32);
    }
}

// parts: the row's chunk partials (global memory or an LDS copy); h0: the histograms of the
// first batch of NB chunks, loaded by hist_batch_load(dm, ws, r, 0, min(kThreads, nchunks), h0).
template <int NB, int NBINS>
__device__ __forceinline__ void topp_range(const Dims& dm, const Samp& sp, int r,
                                           const ChunkPart* parts, float m, double S,
                                           double* s_mass, const Workspace& ws,
                                           HistBatch<NB, NBINS>& h0, TopPRow* s_out = nullptr) {
  const int tid = threadIdx.x;
  __shared__ RedScratch red;
  int emt = INT_MIN;
  for (int c = tid; c < dm.nchunks; c += kThreads)
    if (parts[c].vmax > -INFINITY) emt = max(emt, parts[c].pad[0]);
  const int em = block_max_i(emt, red);
  // row bin B holds the elements with edge em - B (B = NBINS - 1: that edge and below);
  // chunk c's bin j lands in row bin j + (em - edge of chunk c's maximum).  Chunks are added in
  // order, one bin per thread and chunk (the shift is one-to-one below the last bin; a barrier
  // between chunks), so every bin's sum has a fixed order; the last bin's share is summed per
  // thread and reduced.  The histograms are loaded NB chunks at a time.
  constexpr int PT = NBINS / kThreads;
  // each chunk's scale exp((vmax - m) / T) (in 2^-40 units; 0: no mass) and shift em - edge of
  // its maximum, computed once per chunk, in blocks of kThreads chunks
  __shared__ double s_sc[kThreads];
  __shared__ long long s_dc[kThreads];
#pragma unroll
  for (int i = 0; i < PT; ++i) s_mass[tid + i * kThreads] = 0.0;
  double rest = 0.0;
  for (int cb = 0; cb < dm.nchunks; cb += kThreads) {
    __syncthreads();
    const int cc = cb + tid;
    if (cc < dm.nchunks) {  // the scales of this block of chunks
      const ChunkPart p = parts[cc];
      const bool live = p.vmax > -INFINITY;
      s_sc[tid] = live ? exp((double)(p.vmax - m) / (double)sp.temperature) * 0x1p-40 : 0.0;
      s_dc[tid] = live ? (long long)em - p.pad[0] : 0;
    }
    const int ce = min(cb + kThreads, dm.nchunks);
    auto add_batch = [&](const HistBatch<NB, NBINS>& h, int c0) {
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        if (c0 + q >= ce) break;
        __syncthreads();
        const double sc = s_sc[c0 + q - cb];
        if (sc > 0.0) {  // (a chunk with no mass, or whose scale underflows, adds nothing)
          const long long dc = s_dc[c0 + q - cb];
#pragma unroll
          for (int i = 0; i < PT; ++i) {
            const int j = tid + i * kThreads;
            const double v = (double)h[q][i] * sc;
            if (j == NBINS - 1 || j + dc >= NBINS - 1)
              rest += v;
            else
              s_mass[j + dc] += v;
          }
        }
      }
    };
    int c0 = cb;
    if (cb == 0) {
      add_batch(h0, 0);
      c0 = NB;
    }
    for (; c0 < ce; c0 += NB) {
      HistBatch<NB, NBINS> hl;
      hist_batch_load<NB, NBINS>(dm, ws, r, c0, ce, hl);
      add_batch(hl, c0);
    }
  }
  rest = block_sum_d(rest, red);
  if (tid == 0) s_mass[NBINS - 1] = rest;
  __syncthreads();
  if (tid < 64) {
    constexpr int PER = NBINS / 64;
    const int lane = tid;
    double v[PER];
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      v[i] = s_mass[lane * PER + i];
      tot += v[i];
    }
    double inc = tot;  // inclusive scan over lanes, fixed order
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    double cum = __shfl_up(inc, 1);
    if (lane == 0) cum = 0.0;
    const double target = (double)sp.top_p * S;
    int bstar = INT_MAX, last = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      cum += v[i];
      if (cum >= target && bstar == INT_MAX) bstar = lane * PER + i;
      if (v[i] > 0.0) last = lane * PER + i;
    }
    bstar = wave_reduce(bstar, [](int a, int b) { return a < b ? a : b; });
    last = wave_reduce(last, [](int a, int b) { return a > b ? a : b; });
    const bool crossed = bstar != INT_MAX;
    if (!crossed) bstar = last < 0 ? 0 : last;  // rounding kept the total below P S
    // The bin masses differ from the selection's own weights (exp relative to the row maximum,
    // 2^-40 fixed point) by the fp32 exponentials' rounding (< 1e-6 of the mass) and the
    // truncation to 2^-40 (< 2^-40 per element, in both).  When the crossing of P S lies
    // farther than that from both edges of bin bstar, the boundary is in bstar and bstar alone
    // is the candidate range; otherwise its two neighbours are taken too.
    double before = 0.0, through = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (lane * PER + i < bstar) before += v[i];
      if (lane * PER + i <= bstar) through += v[i];
    }
    before = wave_reduce(before, [](double a, double b) { return a + b; });
    through = wave_reduce(through, [](double a, double b) { return a + b; });
    const double eps = 2e-5 * S + (double)dm.V * 0x1p-38;
    const bool single =
        crossed && bstar < NBINS - 1 && before < target - eps && through >= target + eps;
    const int lo = single ? bstar : (bstar > 0 ? bstar - 1 : 0);
    const int hi = single ? bstar : (bstar + 1 < NBINS - 1 ? bstar + 1 : NBINS - 1);
    double above = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane * PER + i < lo) above += v[i];
    above = wave_reduce(above, [](double a, double b) { return a + b; });
    if (lane == 0) {
      TopPRow t;
      t.mass_above = above;
      t.e_hi = em - lo;
      t.e_lo = hi == NBINS - 1 ? INT_MIN : em - hi;
      t.count = 0;
      // every chunk's top edge is at most em, so a code below kCodeFar resolves any edge down
      // to em - (kCodeFar - 1): the codes decide the range when it ends above that
      t.coded = ws.codes != nullptr && hi <= kCodeFar - 1 ? 1 : 0;
      t.em = em;
      t.pad[0] = t.pad[1] = t.pad[2] = 0;
      ws.tprow[r] = t;
      if (s_out) *s_out = t;
    }
  }
}

// Candidates of the boundary bins, appended to the row's list (in no particular order:
// k_topp_select's result does not depend on it).  A chunk gathers its candidates in LDS and
// reserves room in the row's list with one atomic add.  A chunk of a target row also writes its
// kept segment: the index of every element at or above the candidate range's lower edge
// (everything top-p may keep), up to kTopPSegCap, and its count; the final draw reads the
// segments instead of the row.  bf16 rows (fp32 rows take k_topp_row, from edge codes); the
// chunk's logits are read in two halves.
constexpr int kToppChunkCap = 2048;  // candidates one chunk may gather

// Index of row r's kept list (its target row index b * (K + 1) + k), or -1 for a draft row.
__device__ __forceinline__ int kept_list_of(const Dims& dm, int r) {
  if (dm.rows_per_seq == 1) return r;
  const int b = r / dm.rows_per_seq, j = r - b * dm.rows_per_seq;
  return j <= dm.K ? b * (dm.K + 1) + j : -1;
}

template <class E>
__global__ __launch_bounds__(kThreads) void k_topp_cand(const E* __restrict__ tgt,
                                                        const E* __restrict__ drf, Dims dm,
                                                        Samp sp, Workspace ws) {
  const int bid = xcd_contiguous((int)blockIdx.x, dm.rows * dm.nchunks);
  const int r = bid / dm.nchunks;
  const int c = bid - r * dm.nchunks;
  const int tid = threadIdx.x;
  const E* row = row_ptr(dm, tgt, drf, r);
  const TopPRow tr = ws.tprow[r];
  const int e_lo = tr.e_lo, e_hi = tr.e_hi;
  const int kl = kept_list_of(dm, r);
  const float it = sp.inv_t;
  // candidates: (index, logit bits as fp32)
  __shared__ uint2 s_c[kToppChunkCap];
  __shared__ uint32_t s_k[kTopPSegCap];
  __shared__ int s_n, s_nk, s_base;
  if (tid == 0) {
    s_n = 0;
    s_nk = 0;
  }
  auto push = [&](int idx, uint32_t bits, bool cand) {
    if (cand) {
      const int pos = atomicAdd(&s_n, 1);
      if (pos < kToppChunkCap) s_c[pos] = make_uint2((uint32_t)idx, bits);
    }
    if (kl >= 0) {
      const int pos = atomicAdd(&s_nk, 1);
      if (pos < kTopPSegCap) s_k[pos] = (uint32_t)idx;
    }
  };
  {  // the chunk's logits, in two halves
    constexpr int NV = kVecPerThread / 2;
    const int half = dm.chunk_elems / 2;
    __syncthreads();
#pragma unroll 1
    for (int part = 0; part < 2; ++part) {
      uint32_t regs[4 * NV];
      const int f0 = c * dm.chunk_elems + part * half;  // frame index of the half's start
      const int e0 = f0 - load_frame_part<E, NV>(row, dm.V, f0, half, regs, Tr<E>::kNegInfPair);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int h = 0; h < Tr<E>::kPerDword; ++h) {
            const float z = Tr<E>::elem(regs[4 * i + d], h);
            const int e = topp_edge(z, it);
            if (z > -INFINITY && e >= e_lo)
              push(slot_index<E>(e0, i, d, h), __float_as_uint(z), e <= e_hi);
          }
        }
      }
    }
  }
  __syncthreads();
  const int n = s_n, nk = s_nk;
  if (kl >= 0) {  // the segment (a count above kTopPSegCap marks it overflowed)
    const size_t seg = (size_t)kl * dm.nchunks + c;
    if (tid == 0) ws.tkcnt[seg] = nk;
    if (nk <= kTopPSegCap)
      for (int j = tid; j < nk; j += kThreads) ws.tkept[seg * kTopPSegCap + j] = s_k[j];
  }
  if (n == 0) return;
  if (tid == 0)  // a chunk that overflowed its buffer pushes the row past the list capacity
    s_base = atomicAdd(&ws.tprow[r].count, n <= kToppChunkCap ? n : kTopPCandCap + 1);
  __syncthreads();
  if (n <= kToppChunkCap) {
    const int base = s_base;
    uint2* list = ws.tcand + (size_t)r * kTopPCandCap;
    for (int j = tid; j < n && base + j < kTopPCandCap; j += kThreads) list[base + j] = s_c[j];
  }
}

// Order-preserving key of a float (see Tr), with -0 merged into +0.
__device__ __forceinline__ uint32_t float_key(float z) {
  return Tr<float>::canon(Tr<float>::keys_of_dword(__float_as_uint(z)));
}

// Weight of a candidate in 2^-40 fixed point (integer sums: exact whatever their order).
__device__ __forceinline__ unsigned long long topp_weight(uint32_t key, float m, float it) {
  return __float2ull_rz(fast_exp((Tr<float>::key_to_float(key) - m) * it) * 1099511627776.0f);
}

// The exact top-p threshold of a row among its boundary candidates: the largest key v such that
// the mass above the candidate range plus the candidates' mass at keys >= v reaches P * S, by a
// most-significant-digit-first selection on the candidates' keys (8-bit digits, mass-weighted
// bins).  v is the key of the first candidate, in descending order, at which the running mass
// reaches the target; every token at that logit or above is kept.  A row whose candidates
// overflowed the list (or whose candidates' mass does not reach the target, from rounding)
// takes the exact selection by re-reading the row.
template <class E, bool VEC>
__global__ __launch_bounds__(kThreads) void k_topp_select(const E* __restrict__ tgt,
                                                          const E* __restrict__ drf, Dims dm,
                                                          Samp sp, Workspace ws) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ unsigned long long s_buf[kTopPCandCap / 2];  // candidate keys; radix bins on fallback
  __shared__ unsigned long long s_wt[kTopPCandCap];       // candidate weights
  __shared__ unsigned long long s_bins[256];
  __shared__ RedScratch red;
  __shared__ uint32_t s_prefix;
  __shared__ unsigned long long s_need;
  __shared__ uint32_t s_kmin[4], s_kmax[4];
  uint32_t* s_key = reinterpret_cast<uint32_t*>(s_buf);
  RowStat rs = ws.rstat[r];
  const TopPRow tr = ws.tprow[r];
  const float m = rs.m;
  const float it = sp.inv_t;
  const double S = rs.S;
  const int n = tr.count;
  bool fallback = n > kTopPCandCap;
  double Skept = 0.0;
  float thr = -INFINITY;
  if (!fallback) {
    const uint2* list = ws.tcand + (size_t)r * kTopPCandCap;
    unsigned long long tot = 0;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t key = float_key(__uint_as_float(list[i].y));
      const unsigned long long w = topp_weight(key, m, it);
      s_key[i] = key;
      s_wt[i] = w;
      tot += w;
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
    tot = wave_reduce(tot, [](unsigned long long x, unsigned long long y) { return x + y; });
    kmin = wave_reduce(kmin, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
    kmax = wave_reduce(kmax, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
    if (lane_id() == 0) {
      red.u[wave_id()] = tot;
      s_kmin[wave_id()] = kmin;
      s_kmax[wave_id()] = kmax;
    }
    __syncthreads();
    tot = red.u[0] + red.u[1] + red.u[2] + red.u[3];
    kmin = min(min(s_kmin[0], s_kmin[1]), min(s_kmin[2], s_kmin[3]));
    kmax = max(max(s_kmax[0], s_kmax[1]), max(s_kmax[2], s_kmax[3]));
    // the candidates share every key bit above the highest one where kmin and kmax differ, so
    // the digits start at the 8-bit digit holding that bit
    const int hb = kmin == kmax ? 0 : 31 - __clz(kmin ^ kmax);
    const int s0 = (hb / 8) * 8;
    if (tid == 0) s_prefix = s0 + 8 >= 32 ? 0u : (kmin & ~((1u << (s0 + 8)) - 1u));
    const double rem = (double)sp.top_p * S - tr.mass_above;
    unsigned long long need = 1ull;
    if (rem > 0.0) {
      const double q = ceil(rem * 1099511627776.0);
      need = q < 1.8e19 ? (unsigned long long)q : ~0ull;
      if (need == 0ull) need = 1ull;
    }
    if (need > tot) {  // the candidates' mass does not reach the target
      if (tr.e_lo == INT_MIN) {
        thr = -INFINITY;  // rounding: keep every token
        Skept = tr.mass_above + (double)tot * 0x1p-40;
      } else {
        fallback = true;
      }
    } else {
      if (tid == 0) s_need = need;
      for (int shift = s0; shift >= 0; shift -= 8) {
        for (int j = tid; j < 256; j += kThreads) s_bins[j] = 0ull;
        __syncthreads();
        const uint32_t prefix = s_prefix;
        for (int i = tid; i < n; i += kThreads) {
          const uint32_t key = s_key[i];
          if (shift + 8 >= 32 || (key >> (shift + 8)) == (prefix >> (shift + 8)))
            atomicAdd(&s_bins[(key >> shift) & 255u], s_wt[i]);
        }
        __syncthreads();
        if (tid < 64) {  // digits from 255 down: lane L holds 255 - 4L - i, i = 0..3
          const int L = tid;
          unsigned long long bv[4], loc = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bv[i] = s_bins[255 - 4 * L - i];
            loc += bv[i];
          }
          unsigned long long inc = loc;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long y = __shfl_up(inc, o);
            if (L >= o) inc += y;
          }
          const unsigned long long want = s_need;
          unsigned long long cum = inc - loc, before = 0;
          int hit = -1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (hit < 0 && cum + bv[i] >= want) {
              hit = i;
              before = cum;
            }
            cum += bv[i];
          }
          const unsigned long long lanes = __ballot(hit >= 0);
          if (lanes && L == __ffsll((long long)lanes) - 1) {
            s_prefix = prefix | ((uint32_t)(255 - 4 * L - hit) << shift);
            s_need = want - before;
          }
        }
        __syncthreads();
      }
      const uint32_t v = s_prefix;
      thr = Tr<float>::key_to_float(v);
      unsigned long long own = 0;
      for (int i = tid; i < n; i += kThreads)
        if (s_key[i] >= v) own += s_wt[i];
      own = wave_reduce(own, [](unsigned long long x, unsigned long long y) { return x + y; });
      __syncthreads();
      if (lane_id() == 0) red.u[wave_id()] = own;
      __syncthreads();
      Skept = tr.mass_above + (double)(red.u[0] + red.u[1] + red.u[2] + red.u[3]) * 0x1p-40;
    }
  }
  if (fallback) {
    __syncthreads();
    const E* row = row_ptr(dm, tgt, drf, r);
    const uint32_t key =
        radix_select<E, VEC, true>(row, dm.V, m, it, 0u, (double)sp.top_p, s_buf);
    thr = Tr<E>::key_to_float(key);
    Skept = dense_sum<E, VEC>(row, dm.V, m, it, thr, red);
  }
  if (tid == 0) {
    rs.thr = thr;
    rs.S = Skept;
    rs.kind = kRowDense;
    ws.rstat[r] = rs;
  }
}

// ------------------------------------------------------------------------------------------
// k_topp_row (fp32 top-p rows): one workgroup per row does what k_row, k_topp_cand and
// k_topp_select do for bf16 rows, from the chunk partials, the histograms and the edge codes
// that k_chunk wrote: the row's maximum and normaliser, the boundary bracket, a scan of the
// row's codes (two chunks in flight) that collects the candidates' indices in LDS and writes a
// target row's kept segments, the candidates' logits, and the exact threshold by the
// mass-weighted digit selection of k_topp_select (weights recomputed per digit, not stored).
// Rows whose bracket the codes do not reach, or whose candidates overflow, take the exact
// whole-row selection.
// ------------------------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(kThreads, 4) void k_topp_row(const float* __restrict__ tgt,
                                                       const float* __restrict__ drf, Dims dm,
                                                       Samp sp, Workspace ws) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = row_ptr(dm, tgt, drf, r);
  const ChunkPart* parts = ws.parts + (size_t)r * dm.nchunks;
  // candidate indices, then their keys; the boundary mass histogram before; radix bins of the
  // whole-row selection
  __shared__ unsigned long long s_buf[kTopPCandCap / 2];
  __shared__ unsigned long long s_bins[256];
  __shared__ RedScratch red;
  __shared__ TopPRow s_tr;
  __shared__ int s_wn[kThreads / 64];
  constexpr int kPartsCache = 64;  // rows of up to this many chunks keep their partials in LDS
  constexpr int kRowHistBatch = 16;  // chunks per batch of histogram loads
  __shared__ ChunkPart s_parts[kPartsCache];
  __shared__ uint32_t s_prefix;
  __shared__ unsigned long long s_need;
  __shared__ uint32_t s_kmin[4], s_kmax[4];
  constexpr int kBandCache = 1024;  // chunks whose code band is kept in LDS
  __shared__ uint32_t s_band[kBandCache];
  uint32_t* s_key = reinterpret_cast<uint32_t*>(s_buf);
  const float it = sp.inv_t;

  // the first histograms are loaded before anything else (the bracket needs them first), then
  // the chunk partials once, into LDS when the row has few chunks
  HistBatch<kRowHistBatch, kHistBinsF32> h0;
  hist_batch_load<kRowHistBatch, kHistBinsF32>(dm, ws, r, 0, min(kThreads, dm.nchunks), h0);
  const bool pcached = dm.nchunks <= kPartsCache;
  if (pcached && tid < dm.nchunks) s_parts[tid] = parts[tid];
  __syncthreads();
  const ChunkPart* pp = pcached ? s_parts : parts;
  // the row's maximum and normaliser from the chunk partials (fixed order, as k_row)
  float mt = -INFINITY;
  for (int c = tid; c < dm.nchunks; c += kThreads) mt = fmaxf(mt, pp[c].vmax);
  const float m = block_max_f(mt, red);
  double st = 0.0;
  for (int c = tid; c < dm.nchunks; c += kThreads) {
    const ChunkPart p = pp[c];
    if (p.sum > 0.0) st += p.sum * exp((double)(p.vmax - m) / (double)sp.temperature);
  }
  const double S = block_sum_d(st, red);
  topp_range<kRowHistBatch, kHistBinsF32>(dm, sp, r, pp, m, S, reinterpret_cast<double*>(s_buf),
                                          ws, h0,
                            &s_tr);
  __syncthreads();
  const TopPRow tr = s_tr;
  // A chunk's candidates are its codes in [glo, glo + span]: edge = etop - code lies in
  // [e_lo, e_hi] iff etop - e_hi <= code <= etop - e_lo (below kCodeFar for a coded row, so far
  // codes never pass).  Packed glo | span << 16, or kNoBand for a chunk with no finite logit or
  // an empty band.  The bands are kept in LDS, so that the scan reads them without a memory
  // load that would wait on the code loads in flight; rows of more than kBandCache chunks (over
  // 16.7 million logits) take the whole-row selection.
  bool fallback = !tr.coded || dm.nchunks > kBandCache;
  constexpr uint32_t kNoBand = 0xFFFFFFFFu;
  if (!fallback) {
    for (int c = tid; c < dm.nchunks; c += kThreads) {
      const ChunkPart p = parts[c];
      const int etop = p.pad[0];
      const int glo = max(etop - tr.e_hi, 0);
      const int ghi = etop - tr.e_lo;
      s_band[c] = !(p.vmax > -INFINITY) || ghi < glo
                      ? kNoBand
                      : (uint32_t)glo | ((uint32_t)(ghi - glo) << 16);
    }
    __syncthreads();
  }
  // candidates: one list per wave (a quarter of s_key), filled by ballot compaction
  constexpr int kWaveCand = kTopPCandCap / (kThreads / 64);
  uint32_t* wlist = s_key + wave_id() * kWaveCand;
  int wcount = 0;  // uniform in the wave
  if (!fallback) {
    // byte a of chunk c's codes is frame slot c * CH + a, element c * CH - ph + a; thread t
    // holds bytes 16 (t + 256 i) .. + 15 of a chunk
    constexpr int NC = 4;  // 16-byte code vectors per thread and chunk (CH = 16384)
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const uint8_t* rcodes = ws.codes + (size_t)r * dm.nchunks * dm.chunk_elems;
    const int c_ph = row_phase(row);
    auto load_codes = [&](int c, uint32_t(&w)[4 * NC]) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(rcodes + (size_t)c * dm.chunk_elems), (short)0,
          c < dm.nchunks ? dm.chunk_elems : 0, 0x00020000);
#pragma unroll
      for (int i = 0; i < NC; ++i) {  // out of range (c past the row): zeros, never scanned
        const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, i * kThreads * 16, 0);
        w[4 * i + 0] = x.x;
        w[4 * i + 1] = x.y;
        w[4 * i + 2] = x.z;
        w[4 * i + 3] = x.w;
      }
    };
    // Per chunk, each lane first shifts its 64 tests into two hit masks (no branch per code:
    // code k = 4 j + b ends at bit 31 - (k mod 32) of mask k / 32), then the wave appends the
    // hits in rounds, each lane its highest remaining bit per round (a round per hit of the
    // busiest lane).
    auto scan = [&](int c, const uint32_t(&w)[4 * NC]) {
      const uint32_t band = s_band[c];
      if (band == kNoBand) return;
      const uint32_t glo = band & 0xFFFFu;
      const uint32_t n = (band >> 16) + 1u;  // a candidate iff code - glo < n, unsigned
      uint32_t mk[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 4 * NC; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          mk[j >> 3] = shift_in_lt(mk[j >> 3], ((w[j] >> (8 * b)) & 0xFFu) - glo, n);
      const int c0 = c * dm.chunk_elems - c_ph + 16 * tid;
      while (true) {
        const bool has = (mk[0] | mk[1]) != 0u;
        const unsigned long long m = __ballot(has);
        if (!m) break;
        const int k = mk[0] ? __builtin_clz(mk[0]) : 32 + __builtin_clz(mk[1] | 1u);
        if (mk[0])
          mk[0] &= ~(0x80000000u >> k);
        else
          mk[1] &= ~(0x80000000u >> (k - 32));
        const int pos = lane_rank(m, wcount);
        if (has && pos < kWaveCand) wlist[pos] = (uint32_t)(c0 + kThreads * 16 * (k >> 4) + (k & 15));
        wcount += __popcll(m);
      }
    };
    // four chunks in flight: each buffer is refilled with the chunk four ahead once scanned
    uint32_t wa[4 * NC], wb[4 * NC], wc[4 * NC], wd[4 * NC];
    // issued in chunk order (no reordering by the scheduler), so that the loop's first scan
    // waits for the oldest loads only
    load_codes(0, wa);
    __builtin_amdgcn_sched_barrier(0);
    load_codes(1, wb);
    __builtin_amdgcn_sched_barrier(0);
    load_codes(2, wc);
    __builtin_amdgcn_sched_barrier(0);
    load_codes(3, wd);
    __builtin_amdgcn_sched_barrier(0);
    // (no early exit: one back edge, so the loop's waits stay those of the steady state; loads
    // past the row's end read nothing)
    for (int c = 0; c < dm.nchunks; c += 4) {
      scan(c, wa);
      load_codes(c + 4, wa);
      if (c + 1 < dm.nchunks) scan(c + 1, wb);
      load_codes(c + 5, wb);
      if (c + 2 < dm.nchunks) scan(c + 2, wc);
      load_codes(c + 6, wc);
      if (c + 3 < dm.nchunks) scan(c + 3, wd);
      load_codes(c + 7, wd);
    }
    if (lane_id() == 0) s_wn[wave_id()] = wcount;
    __syncthreads();
    for (int w = 0; w < kThreads / 64; ++w)
      if (s_wn[w] > kWaveCand) fallback = true;
  }
  double Skept = 0.0;
  float thr = -INFINITY;
  if (!fallback) {
    // the wave lists in place, one after another: entry i of list w at w * kWaveCand + i
    int nw[kThreads / 64];
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) nw[w] = s_wn[w];
    auto for_cands = [&](auto&& f) {
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w)
        for (int i = tid; i < nw[w]; i += kThreads) f(w * kWaveCand + i);
    };
    // the candidates' logits: every load issued before the first is used (at most
    // kWaveCand / kThreads per thread and list)
    constexpr int PL = kWaveCand / kThreads;
    float zc[kThreads / 64][PL];
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w)
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const int i = tid + k * kThreads;
        zc[w][k] = i < nw[w] ? row[s_key[w * kWaveCand + i]] : 0.0f;
      }
    unsigned long long tot = 0;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w)
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const int i = tid + k * kThreads;
        if (i < nw[w]) {  // as keys
          const uint32_t key = float_key(zc[w][k]);
          s_key[w * kWaveCand + i] = key;
          tot += topp_weight(key, m, it);
          kmin = min(kmin, key);
          kmax = max(kmax, key);
        }
      }
    tot = wave_reduce(tot, [](unsigned long long x, unsigned long long y) { return x + y; });
    kmin = wave_reduce(kmin, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
    kmax = wave_reduce(kmax, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
    if (lane_id() == 0) {
      red.u[wave_id()] = tot;
      s_kmin[wave_id()] = kmin;
      s_kmax[wave_id()] = kmax;
    }
    __syncthreads();
    tot = red.u[0] + red.u[1] + red.u[2] + red.u[3];
    kmin = min(min(s_kmin[0], s_kmin[1]), min(s_kmin[2], s_kmin[3]));
    kmax = max(max(s_kmax[0], s_kmax[1]), max(s_kmax[2], s_kmax[3]));
    // the candidates share every key bit above the highest one where kmin and kmax differ, so
    // the digits start at the 8-bit digit holding that bit
    const int hb = kmin == kmax ? 0 : 31 - __clz(kmin ^ kmax);
    const int s0 = (hb / 8) * 8;
    const double rem = (double)sp.top_p * S - tr.mass_above;
    unsigned long long need = 1ull;
    if (rem > 0.0) {
      const double q = ceil(rem * 1099511627776.0);
      need = q < 1.8e19 ? (unsigned long long)q : ~0ull;
      if (need == 0ull) need = 1ull;
    }
    __syncthreads();  // every thread has read red and the key bounds
    if (need > tot) {  // the candidates' mass does not reach the target (rounding)
      fallback = true;
    } else {
      if (tid == 0) {
        s_need = need;
        s_prefix = s0 + 8 >= 32 ? 0u : (kmin & ~((1u << (s0 + 8)) - 1u));
      }
      for (int shift = s0; shift >= 0; shift -= 8) {
        s_bins[tid] = 0ull;
        __syncthreads();
        const uint32_t prefix = s_prefix;
        for_cands([&](int i) {
          const uint32_t key = s_key[i];
          if (shift + 8 >= 32 || (key >> (shift + 8)) == (prefix >> (shift + 8)))
            atomicAdd(&s_bins[(key >> shift) & 255u], topp_weight(key, m, it));
        });
        __syncthreads();
        if (tid < 64) {  // digits from 255 down: lane L holds 255 - 4L - i, i = 0..3
          const int L = tid;
          unsigned long long bv[4], loc = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bv[i] = s_bins[255 - 4 * L - i];
            loc += bv[i];
          }
          unsigned long long inc = loc;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long y = __shfl_up(inc, o);
            if (L >= o) inc += y;
          }
          const unsigned long long want = s_need;
          unsigned long long cum = inc - loc, before = 0;
          int hit = -1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (hit < 0 && cum + bv[i] >= want) {
              hit = i;
              before = cum;
            }
            cum += bv[i];
          }
          const unsigned long long lanes = __ballot(hit >= 0);
          if (lanes && L == __ffsll((long long)lanes) - 1) {
            s_prefix = prefix | ((uint32_t)(255 - 4 * L - hit) << shift);
            s_need = want - before;
          }
        }
        __syncthreads();
      }
      const uint32_t v = s_prefix;
      thr = Tr<float>::key_to_float(v);
      unsigned long long own = 0;
      for_cands([&](int i) {
        if (s_key[i] >= v) own += topp_weight(s_key[i], m, it);
      });
      own = wave_reduce(own, [](unsigned long long x, unsigned long long y) { return x + y; });
      if (lane_id() == 0) red.u[wave_id()] = own;
      __syncthreads();
      Skept = tr.mass_above + (double)(red.u[0] + red.u[1] + red.u[2] + red.u[3]) * 0x1p-40;
    }
  }
  if (fallback) {
    __syncthreads();
    const uint32_t key =
        radix_select<float, VEC, true>(row, dm.V, m, it, 0u, (double)sp.top_p, s_buf);
    thr = Tr<float>::key_to_float(key);
    Skept = dense_sum<float, VEC>(row, dm.V, m, it, thr, red);
  }
  if (tid == 0) {
    RowStat out;
    out.m = m;
    out.thr = thr;
    out.S = Skept;
    out.argmax = -1;
    out.nkept = -1;
    out.kind = kRowDense;
    out.pad = 0;
    ws.rstat[r] = out;
  }
}

// ------------------------------------------------------------------------------------------
// k_row: one workgroup per row.  Produces RowStat (m, thr, S) from the chunk partials; top-k
// above the compact limit and top-p select their thresholds by re-reading the row.
// ------------------------------------------------------------------------------------------
template <class E, bool VEC>
__global__ __launch_bounds__(kThreads) void k_row(const E* __restrict__ tgt,
                                                  const E* __restrict__ drf, Dims dm, Samp sp,
                                                  Workspace ws) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const E* row = row_ptr(dm, tgt, drf, r);
  const ChunkPart* parts = ws.parts + (size_t)r * dm.nchunks;
  __shared__ RedScratch red;
  __shared__ unsigned long long s_bins[2048];  // radix bins
  __shared__ float s_m;
  __shared__ int s_argmax;
  __shared__ double s_S;

  // Row maximum (and the lowest index holding it), then the normaliser, over the chunk
  // partials: threads take chunks in a fixed order and combine in a fixed tree.
  float mt = -INFINITY;
  int at = INT_MAX;
  for (int c = tid; c < dm.nchunks; c += kThreads) {
    const ChunkPart p = parts[c];
    if (p.vmax > mt) {  // chunks of one thread ascend, so the first maximum wins
      mt = p.vmax;
      at = p.argmax;
    }
  }
  const float mrow = block_max_f(mt, red);
  const int am = block_min_i(mt == mrow ? at : INT_MAX, red);
  double st = 0.0;
  if (!sp.greedy) {
    for (int c = tid; c < dm.nchunks; c += kThreads) {
      const ChunkPart p = parts[c];
      if (p.sum > 0.0) st += p.sum * exp((double)(p.vmax - mrow) / (double)sp.temperature);
    }
  }
  const double Srow = sp.greedy ? 0.0 : block_sum_d(st, red);
  if (tid == 0) {
    s_m = mrow;
    s_argmax = am;
    s_S = Srow;
  }
  __syncthreads();
  const float m = s_m;
  RowStat out;
  out.m = m;
  out.argmax = -1;
  out.nkept = -1;
  out.pad = 0;

  if (sp.greedy) {
    if (tid == 0) {
      out.thr = -INFINITY;
      out.S = 1.0;
      out.argmax = s_argmax;
      out.nkept = 1;
      out.kind = kRowGreedy;
      ws.rstat[r] = out;
    }
    return;
  }

  const float it = sp.inv_t;
  if (sp.topp_hist) {
    // top-p without top-k: locate the boundary bin of the merged mass histogram; the exact
    // threshold is taken among the boundary candidates by k_topp_select
    constexpr int NBINS = sizeof(E) == 4 ? kHistBinsF32 : kHistBins;
    HistBatch<2, NBINS> h0;
    hist_batch_load<2, NBINS>(dm, ws, r, 0, min(kThreads, dm.nchunks), h0);
    topp_range<2, NBINS>(dm, sp, r, parts, m, s_S, reinterpret_cast<double*>(s_bins), ws, h0);
    if (tid == 0) {
      out.thr = -INFINITY;
      out.S = s_S;
      out.kind = kRowDense;
      ws.rstat[r] = out;
    }
    return;
  }
  uint32_t lower_key = 0;  // selection threshold key (0: none)

  // Whole-row path: exact selections by re-reading the row.
  const bool topk_on = sp.top_k > 0 && sp.top_k < dm.V;
  if (topk_on)
    lower_key = radix_select<E, VEC, false>(row, dm.V, m, it, 0u, (double)sp.top_k, s_bins);
  if (sp.top_p < 1.0f)
    lower_key =
        radix_select<E, VEC, true>(row, dm.V, m, it, lower_key, (double)sp.top_p, s_bins);
  const bool trunc = topk_on || sp.top_p < 1.0f;
  const float thr = (trunc && lower_key) ? Tr<E>::key_to_float(lower_key) : -INFINITY;
  double S = trunc ? dense_sum<E, VEC>(row, dm.V, m, it, thr, red) : s_S;
  if (tid == 0) {
    out.thr = thr;
    out.S = S;
    out.kind = kRowDense;
    ws.rstat[r] = out;
  }
}

// Unnormalised weight of a logit in a row's kept set: exp((z - m) / T) in fp32.
__device__ __forceinline__ float kept_exp(float z, const RowStat& rs, float it) {
  return z >= rs.thr ? fast_exp((z - rs.m) * it) : 0.0f;
}

struct Outs {
  const int32_t* drafts;  // [B, K]
  const float* uni;       // [B, K+1]
  int32_t* tokens;        // [B, K+1]
  int32_t* n;             // [B]
  float* a;               // [B, K] or null
  float* q;               // [B, K] or null
  float* p;               // [B, K] or null
};

// Accept tests of sequence b by one wave: lane k handles position k (Chen et al. notes, A2:
// accept x~_k with probability min(1, q/p); lenience scales the comparison, App. F of the
// Leviathan blog).  Writes a/q/p, the accepted drafts, the -1 padding after position n and n;
// position n itself is written by the final draw.  Returns n in every lane.
// rstat(r): the statistics of row r (from memory, or from a caller's copy in LDS);
// zx(k, x, zt, zd): the logits of target row k and draft row k at token x (0 <= x < V); x_pre:
// this lane's draft token when the caller loaded it already (lane k, k < 64), else -2
template <class E, class RS, class ZX>
__device__ int seq_accept_wave(const E* __restrict__ tgt, const E* __restrict__ drf,
                               const Dims& dm, const Samp& sp, const Workspace& ws,
                               const Outs& o, int b, RS&& rstat, ZX&& zx, int x_pre) {
  const int lane = lane_id();
  const int K = dm.K, V = dm.V;
  const double T = (double)sp.temperature;
  int n = K;
  bool found = false;
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int k = k0 + lane;
    bool rej = false;
    if (k < K) {
      const int x = (k0 == 0 && x_pre != -2) ? x_pre : o.drafts[(size_t)b * K + k];
      const RowStat rt = rstat(target_row(dm, b, k));
      const RowStat rd = rstat(draft_row(dm, b, k));
      double q = 0.0, p = 0.0, a;
      const MentorSol* ms = sp.mentor ? ws.ment + (size_t)b * K + k : nullptr;
      if (ms && ms->mode != kMentorLossless) {  // mentored decoding: r at the draft token
        q = ms->qx;
        p = ms->px;
        a = ms->a;
      } else {
        if (x >= 0 && x < V) {
          if (sp.greedy) {
            q = (x == rt.argmax) ? 1.0 : 0.0;
            p = (x == rd.argmax) ? 1.0 : 0.0;
          } else {
            float zt, zd;
            zx(k, x, zt, zd);
            if (zt >= rt.thr) q = exp(((double)zt - (double)rt.m) / T) / rt.S;
            if (zd >= rd.thr) p = exp(((double)zd - (double)rd.m) / T) / rd.S;
          }
        }
        if (p > 0.0) {
          a = q / ((double)sp.lenience * p);
          a = a < 1.0 ? a : 1.0;
        } else {
          a = q > 0.0 ? 1.0 : 0.0;
        }
      }
      rej = !((double)o.uni[(size_t)b * (K + 1) + k] < a);
      if (o.a) o.a[(size_t)b * K + k] = (float)a;
      if (o.q) o.q[(size_t)b * K + k] = (float)q;
      if (o.p) o.p[(size_t)b * K + k] = (float)p;
    }
    const unsigned long long mask = __ballot(rej);
    if (!found && mask) {
      n = k0 + __ffsll((long long)mask) - 1;
      found = true;
    }
  }
  for (int j = lane; j <= K; j += 64) {
    if (j < n) o.tokens[(size_t)b * (K + 1) + j] = o.drafts[(size_t)b * K + j];
    if (j > n) o.tokens[(size_t)b * (K + 1) + j] = -1;
  }
  if (lane == 0) o.n[b] = n;
  return n;
}

// The same with the statistics from the workspace, each lane's position's loaded once into
// `ls` (lane k: target row k for k <= K, draft row k for k < K; positions past the first 64 are
// loaded where the scan reaches them), so that the statistics of the final row pair come from
// lane n (final_row_stats) instead of a further load after the scan.
struct LaneStats {
  RowStat t, d;
};

template <class E>
__device__ int seq_accept_wave(const E* __restrict__ tgt, const E* __restrict__ drf,
                               const Dims& dm, const Samp& sp, const Workspace& ws,
                               const Outs& o, int b, LaneStats& ls) {
  const int l = lane_id(), K = dm.K;
  if (l <= K) ls.t = ws.rstat[target_row(dm, b, l)];
  if (l < K) ls.d = ws.rstat[draft_row(dm, b, l)];
  return seq_accept_wave(
      tgt, drf, dm, sp, ws, o, b,
      [&](int r) {
        if (l <= K && r == target_row(dm, b, l)) return ls.t;
        if (l < K && r == draft_row(dm, b, l)) return ls.d;
        return ws.rstat[r];
      },
      [&](int k, int x, float& zt, float& zd) {
        zt = load_logit(row_ptr(dm, tgt, drf, target_row(dm, b, k)), x);
        zd = load_logit(row_ptr(dm, tgt, drf, draft_row(dm, b, k)), x);
      },
      -2);
}

// Lane l's copy of a RowStat (l the same in every lane).
__device__ __forceinline__ RowStat lane_rowstat(const RowStat& s, int l) {
  typedef int i8 __attribute__((ext_vector_type(8)));
  static_assert(sizeof(RowStat) == sizeof(i8), "RowStat is eight dwords");
  const i8 v = __builtin_bit_cast(i8, s);
  i8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = __builtin_amdgcn_readlane(v[j], l);
  return __builtin_bit_cast(RowStat, r);
}

// The statistics of target row n and of the final draw's other row (draft row n, or target row
// n again for the bonus draw), from the lanes of seq_accept_wave when n < 64.
__device__ __forceinline__ void final_row_stats(const Dims& dm, const Workspace& ws, int b, int n,
                                                const LaneStats& ls, RowStat& rt, RowStat& rd) {
  rt = n < 64 ? lane_rowstat(ls.t, n) : ws.rstat[target_row(dm, b, n)];
  rd = n >= dm.K ? rt : n < 64 ? lane_rowstat(ls.d, n) : ws.rstat[draft_row(dm, b, n)];
}

// A top-p target row's kept segments (bf16) hold every element at or above the candidate range's
// lower edge; they hold the whole kept set {z >= thr} iff none overflowed and the threshold's
// edge is inside that range (a row whose boundary selection re-read the row may have a threshold
// below it).  fp32 rows: see below.  Called by a whole wave; the same answer in every lane.
__device__ __forceinline__ bool kept_list_complete(const Dims& dm, const Samp& sp,
                                                   const Workspace& ws, int b, int n,
                                                   const RowStat& rt) {
  const TopPRow tr = ws.tprow[target_row(dm, b, n)];
  if (ws.codes) {
    // fp32 rows carry edge codes instead of segments: the draw scans them, which finds every
    // kept element when each has a code below kCodeFar, i.e. when the threshold's edge is at
    // most kCodeFar - 1 steps below the row maximum's (and every chunk maximum is at most that)
    return rt.thr > -INFINITY && topp_edge(rt.thr, sp.inv_t) >= tr.em - (kCodeFar - 1);
  }
  bool ok = tr.e_lo == INT_MIN || topp_edge(rt.thr, sp.inv_t) >= tr.e_lo;
  const int* cnt = ws.tkcnt + (size_t)(b * (dm.K + 1) + n) * dm.nchunks;
  for (int c = lane_id(); c < dm.nchunks; c += 64) ok = ok && cnt[c] <= kTopPSegCap;
  return __ballot(!ok) == 0ull;
}

// ------------------------------------------------------------------------------------------
// k_seq: one wave per sequence.  Accept tests, first rejection, and the final draw when the
// final row is greedy or compact.
// ------------------------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(kSeqThreads) void k_seq(const E* __restrict__ tgt,
                                                     const E* __restrict__ drf, Dims dm,
                                                     Samp sp, Workspace ws, Outs o) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int K = dm.K;
  const float* uni = o.uni;
  int32_t* out_tokens = o.tokens;
  __shared__ double s_w[kKeptCap];
  __shared__ double s_q[kKeptCap];

  LaneStats ls;
  const int n = seq_accept_wave(tgt, drf, dm, sp, ws, o, b, ls);
  // target row n, and the draft row of position n (the target row again for the bonus draw)
  RowStat rt, rd_n;
  final_row_stats(dm, ws, b, n, ls, rt, rd_n);
  SeqState st;
  st.n = n;
  st.need_dense = 0;
  st.fallback = 0;
  st.need_list = 0;
  int tok = -1;
  if (rt.kind == kRowGreedy) {
    // one-hot q and p: the residual is one-hot at the target argmax or empty (then q is used)
    tok = rt.argmax;
  } else if (rt.kind == kRowCompact) {
    const float it = sp.inv_t;
    const int nk = rt.nkept;
    const uint2* kept = ws.kept + (size_t)target_row(dm, b, n) * kKeptCap;
    const bool resid = n < K;
    const RowStat rd = rd_n;
    const E* drow = resid ? row_ptr(dm, tgt, drf, draft_row(dm, b, n)) : nullptr;
    for (int j = lane; j < nk; j += kSeqThreads) {
      const uint2 e = kept[j];
      const double q = (double)fast_exp((__uint_as_float(e.y) - rt.m) * it) / rt.S;
      double w = q;
      if (resid) {
        const double p = (double)kept_exp(load_logit(drow, (int)e.x), rd, it) / rd.S;
        w = q - p > 0.0 ? q - p : 0.0;
      }
      s_q[j] = q;
      s_w[j] = w;
    }
    __syncthreads();
    if (lane == 0) {
      double W = 0.0;
      for (int j = 0; j < nk; ++j) W += s_w[j];
      const double* wv = s_w;
      if (!(W > 0.0)) {
        st.fallback = 1;
        W = 0.0;
        for (int j = 0; j < nk; ++j) W += s_q[j];
        wv = s_q;
      }
      const double target = (double)uni[(size_t)b * (K + 1) + K] * W;
      double cum = 0.0;
      int pick = -1, last_pos = -1;
      for (int j = 0; j < nk; ++j) {
        if (wv[j] > 0.0) last_pos = j;
        cum += wv[j];
        if (pick < 0 && cum > target) pick = j;
      }
      if (pick < 0) pick = last_pos;
      if (pick < 0) pick = 0;
      tok = (int)kept[pick].x;
    }
  } else if (sp.topp_hist && kept_list_complete(dm, sp, ws, b, n, rt)) {
    st.need_list = 1;  // top-p: the draw reads the target row's kept list
  } else {
    st.need_dense = 1;
  }
  if (lane == 0) {
    if (!st.need_dense && !st.need_list) out_tokens[(size_t)b * (K + 1) + n] = tok;
    ws.seq[b] = st;
    if (st.need_dense || st.need_list) {  // read by the final draw's kernels with the state
      ws.dstat[2 * b] = rt;
      ws.dstat[2 * b + 1] = rd_n;
    }
  }
}

// Weight of element z of the final row pair: (q - p)_+ (residual) or q (bonus / fallback).
__device__ __forceinline__ double final_weight(float zt, float zd, const RowStat& rt,
                                               const RowStat& rd, bool resid, bool use_q,
                                               float it) {
  const double q = (double)kept_exp(zt, rt, it) / rt.S;
  if (!resid || use_q) return q;
  const double p = (double)kept_exp(zd, rd, it) / rd.S;
  return q - p > 0.0 ? q - p : 0.0;
}

// Load elements [e0, e0 + EPV) of a row as floats; past the row end: -inf (weight 0).
template <class E, bool VEC>
__device__ __forceinline__ void load_vec_f(const E* row, int V, int e0, float (&z)[Tr<E>::kEpv]) {
  constexpr int EPV = Tr<E>::kEpv;
  if constexpr (VEC) {
    if (e0 < V) {
      const uint4 x = *reinterpret_cast<const uint4*>(row + e0);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int h = 0; h < Tr<E>::kPerDword; ++h)
          z[d * Tr<E>::kPerDword + h] = Tr<E>::elem(w[d], h);
    } else {
#pragma unroll
      for (int e = 0; e < EPV; ++e) z[e] = -INFINITY;
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPV; ++e) z[e] = (e0 + e < V) ? load_logit(row, e0 + e) : -INFINITY;
  }
}

// Weights of the final draw for one element pair, in fp32 with the normalisers' reciprocals
// taken once per row: w = max(0, q - p) (the residual, Theorem 1) and q.  Sums over them run in
// fp64 (per 16-byte vector in fp32 first).
struct DrawRows {
  RowStat rt, rd;
  float inv_st, inv_sd;
  bool resid;
};

__device__ __forceinline__ void draw_weights(float zt, float zd, const DrawRows& g, float it,
                                             float& w, float& q) {
  q = kept_exp(zt, g.rt, it) * g.inv_st;
  w = q;
  if (g.resid) w = fmaxf(q - kept_exp(zd, g.rd, it) * g.inv_sd, 0.0f);
}

// From the final draw's row statistics that k_seq stored for sequence b (rt, rd).
__device__ __forceinline__ DrawRows draw_rows(const Dims& dm, int n, const RowStat& rt,
                                              const RowStat& rd) {
  DrawRows g;
  g.resid = n < dm.K;
  g.rt = rt;
  g.rd = g.resid ? rd : rt;
  g.inv_st = (float)(1.0 / g.rt.S);
  g.inv_sd = (float)(1.0 / g.rd.S);
  return g;
}


// NV 16-byte vectors per thread from a row.  STRIDED: vector i of thread t at element
// base + (t + 256 i) * EPV; otherwise a contiguous run, vector i at base + i * EPV.  With VEC the
// loads are range-checked buffer loads, so no load sits behind a branch: elements at or past
// `end` read as 0 and the caller must not use them.  Without VEC they read as -inf.  `end` must
// be the same in every lane (it sets the buffer's range).
template <class E, bool VEC, int NV, bool STRIDED>
__device__ __forceinline__ void load_vecs(const E* __restrict__ row, int end, int base,
                                          uint32_t (&regs)[4 * NV]) {
  constexpr int EPV = Tr<E>::kEpv;
  constexpr uint32_t kNegInf = Tr<E>::kNegInfPair;
  const int t = STRIDED ? (int)threadIdx.x : 0;
  if constexpr (VEC) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<E*>(row), (short)0, end * (int)sizeof(E), 0x00020000);
    const int voff = (base + t * EPV) * (int)sizeof(E);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int step = STRIDED ? kThreads * EPV : EPV;
      const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, i * step * (int)sizeof(E), 0);
      regs[4 * i + 0] = x.x;
      regs[4 * i + 1] = x.y;
      regs[4 * i + 2] = x.z;
      regs[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = base + (t + (STRIDED ? kThreads * i : i)) * EPV;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t w = 0;
#pragma unroll
        for (int h = 0; h < Tr<E>::kPerDword; ++h) {
          const int idx = e + d * Tr<E>::kPerDword + h;
          const uint32_t bits = idx < end ? Tr<E>::bits_of(row[idx])
                                          : ((Tr<E>::kPerDword == 2) ? 0xFF80u : kNegInf);
          w |= bits << (16 * h * (Tr<E>::kPerDword == 2));
        }
        regs[4 * i + d] = w;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// The final draw of a top-p sequence from the kept segments of its target row n (every element
// top-p may keep, per chunk, in no particular order): q = exp((z - m) / T) / S on the kept set
// {z >= thr}, p at the same index from the draft row (the residual (q - p)_+ is zero wherever q
// is), or q alone for the bonus draw.  Weights are taken in 2^-62 fixed point, so that every
// sum is exact whatever the order of its terms; the token is the smallest index whose
// cumulative weight in index order exceeds u * W.
//   final_lpart  (in k_final_partial, one workgroup per segment): each segment's masses
//   final_lpick  (in k_final_pick, one workgroup per sequence): the segment holding u * W from
//                the masses in chunk order, then the index inside it by two digits (bins of 256
//                indices, then single indices)
// ------------------------------------------------------------------------------------------
// The weights from the two logits at an index (zd unused for the bonus draw).
__device__ __forceinline__ void list_weights_z(float z, float zd, const RowStat& rt,
                                               const RowStat& rd, bool resid, float it,
                                               unsigned long long& wq, unsigned long long& ww) {
  const double q = z >= rt.thr ? (double)fast_exp((z - rt.m) * it) / rt.S : 0.0;
  double w = q;
  if (resid && q > 0.0) {
    const double p = (double)kept_exp(zd, rd, it) / rd.S;
    w = q - p > 0.0 ? q - p : 0.0;
  }
  wq = (unsigned long long)(q * 0x1p62);
  ww = (unsigned long long)(w * 0x1p62);
}

// Both logits are loaded before either is used (one memory round trip, not two).
template <class E>
__device__ __forceinline__ void list_weights(int idx, const RowStat& rt, const RowStat& rd,
                                             bool resid, const E* __restrict__ trow,
                                             const E* __restrict__ drow, float it,
                                             unsigned long long& wq, unsigned long long& ww) {
  const float z = load_logit(trow, idx);
  const float zd = resid ? load_logit(drow, idx) : 0.0f;
  list_weights_z(z, zd, rt, rd, resid, it, wq, ww);
}

template <class E>
__device__ void final_lpart(const E* __restrict__ tgt, const E* __restrict__ drf, const Dims& dm,
                            const Samp& sp, const Workspace& ws, int b, int c, const SeqState& st,
                            const RowStat& rt, const RowStat& rd) {
  const int K = dm.K, n = st.n;
  const bool resid = n < K;
  const size_t seg = (size_t)(b * (K + 1) + n) * dm.nchunks + c;
  const int cnt = ws.tkcnt[seg];
  const uint32_t* list = ws.tkept + seg * kTopPSegCap;
  const E* trow = row_ptr(dm, tgt, drf, target_row(dm, b, n));
  const E* drow = resid ? row_ptr(dm, tgt, drf, draft_row(dm, b, n)) : nullptr;
  unsigned long long W = 0, Q = 0;
  for (int e = threadIdx.x; e < cnt; e += kThreads) {
    unsigned long long wq, ww;
    list_weights<E>((int)list[e], rt, rd, resid, trow, drow, sp.inv_t, wq, ww);
    W += ww;
    Q += wq;
  }
  auto add = [](unsigned long long x, unsigned long long y) { return x + y; };
  W = wave_reduce(W, add);
  Q = wave_reduce(Q, add);
  __shared__ unsigned long long s_wq[2][kThreads / 64];
  if (lane_id() == 0) {
    s_wq[0][wave_id()] = W;
    s_wq[1][wave_id()] = Q;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    ws.lpart[(size_t)b * dm.nchunks + c] =
        make_ulonglong2(s_wq[0][0] + s_wq[0][1] + s_wq[0][2] + s_wq[0][3],
                        s_wq[1][0] + s_wq[1][1] + s_wq[1][2] + s_wq[1][3]);
}

// One wave: the first of PER * 64 bins, in order, at which the running mass exceeds rem (bins
// without mass never qualify); if rounding leaves none, the last bin with mass.  Returns the bin
// and sets before to the mass of the bins ahead of it.
template <int PER>
__device__ int wave_pick_bin(const unsigned long long* bins, double rem,
                             unsigned long long& before) {
  const int lane = lane_id();
  unsigned long long bv[PER], loc = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    bv[i] = bins[PER * lane + i];
    loc += bv[i];
  }
  unsigned long long inc = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  unsigned long long cum = inc - loc, bf = 0, bl = 0;
  int hit = -1, last = -1;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (hit < 0 && bv[i] > 0 && (double)(cum + bv[i]) > rem) {
      hit = i;
      bf = cum;
    }
    if (bv[i] > 0) {
      last = i;
      bl = cum;
    }
    cum += bv[i];
  }
  const unsigned long long hl = __ballot(hit >= 0), pl = __ballot(last >= 0);
  if (hl) {
    const int f = __ffsll((long long)hl) - 1;
    before = __shfl(bf, f);
    return __shfl(PER * lane + hit, f);
  }
  const int f = pl ? 63 - __clzll((long long)pl) : 0;
  before = pl ? __shfl(bl, f) : 0ull;
  return pl ? __shfl(PER * lane + last, f) : 0;
}

// The segment (chunk) holding u * W of a list draw: wave 0 scans the segments' masses in chunk
// order.  Called by the whole workgroup; returns the chunk, the mass left to cover inside it, and
// whether q replaces the residual (no residual, or a residual without mass).
__device__ int pick_list_chunk(const Dims& dm, const Workspace& ws, const float* __restrict__ uni,
                               int b, bool resid, double& rem_out, bool& use_q_out) {
  const int tid = threadIdx.x, lane = lane_id();
  const int K = dm.K;
  __shared__ int s_c;
  __shared__ double s_rem;
  __shared__ int s_useq;
  if (tid < 64) {
    const ulonglong2* lp = ws.lpart + (size_t)b * dm.nchunks;
    unsigned long long W = 0, Q = 0;
    for (int c = lane; c < dm.nchunks; c += 64) {
      W += lp[c].x;
      Q += lp[c].y;
    }
    auto add = [](unsigned long long x, unsigned long long y) { return x + y; };
    W = wave_reduce(W, add);
    Q = wave_reduce(Q, add);
    const bool use_q = !resid || W == 0ull;
    double rem = (double)uni[(size_t)b * (K + 1) + K] * (double)(use_q ? Q : W);
    unsigned long long carry = 0;
    int pick = -1, last = -1;
    unsigned long long before_last = 0;
    double rem_pick = 0.0;
    for (int c0 = 0; c0 < dm.nchunks && pick < 0; c0 += 64) {
      const int c = c0 + lane;
      const unsigned long long m = c < dm.nchunks ? (use_q ? lp[c].y : lp[c].x) : 0ull;
      unsigned long long inc = m;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      const unsigned long long cb = carry + inc - m;  // mass of the chunks ahead of c
      const unsigned long long hl = __ballot(m > 0 && (double)(cb + m) > rem);
      const unsigned long long pl = __ballot(m > 0);
      if (hl) {
        const int f = __ffsll((long long)hl) - 1;
        pick = c0 + f;
        rem_pick = rem - (double)__shfl(cb, f);
      } else if (pl) {
        const int f = 63 - __clzll((long long)pl);
        last = c0 + f;
        before_last = __shfl(cb, f);
      }
      carry += __shfl(inc, 63);
    }
    if (pick < 0) {  // rounding left u W at or past the total: the last chunk with mass
      pick = last < 0 ? 0 : last;
      rem_pick = rem - (double)before_last;
    }
    if (lane == 0) {
      s_c = pick;
      s_rem = rem_pick;
      s_useq = use_q ? 1 : 0;
    }
  }
  __syncthreads();
  rem_out = s_rem;
  use_q_out = s_useq != 0;
  return s_c;
}

// The index of the pick inside a chunk from its entries' positions a (relative to the chunk's
// first slot, below 32768) and weights: the first of 128 bins of 256 positions whose running
// mass passes rem, then the position inside it; add(a, w) is called by the caller for every
// entry in each of the two passes (pass 0: bins of 256, pass 1: positions of bin d1).
template <class F>
__device__ int pick_in_chunk(double rem, F&& entries) {
  const int tid = threadIdx.x, lane = lane_id();
  __shared__ unsigned long long s_bins[256];
  __shared__ int s_d1;
  __shared__ double s_rem;
  s_bins[tid] = 0ull;
  __syncthreads();
  entries(-1, [&](int a, unsigned long long w) {
    if (w) atomicAdd(&s_bins[a >> 8], w);
  });
  __syncthreads();
  if (tid < 64) {
    unsigned long long before;
    const int d1 = wave_pick_bin<4>(s_bins, rem, before);
    if (lane == 0) {
      s_d1 = d1;
      s_rem = rem - (double)before;
    }
  }
  __syncthreads();
  const int d1 = s_d1;
  rem = s_rem;
  s_bins[tid] = 0ull;
  __syncthreads();
  entries(d1, [&](int a, unsigned long long w) {
    if (w && (a >> 8) == d1) atomicAdd(&s_bins[a & 255], w);
  });
  __syncthreads();
  int pick = 0;
  if (tid < 64) {
    unsigned long long before;
    pick = (d1 << 8) + wave_pick_bin<4>(s_bins, rem, before);
  }
  return pick;  // valid in wave 0
}

template <class E>
__device__ void final_lpick(const E* __restrict__ tgt, const E* __restrict__ drf, const Dims& dm,
                            const Samp& sp, const Workspace& ws, const float* __restrict__ uni,
                            int32_t* __restrict__ out_tokens, int b, const SeqState& st,
                            const RowStat& rt, const RowStat& rd) {
  const int tid = threadIdx.x;
  const int K = dm.K, n = st.n;
  const bool resid = n < K;
  constexpr int PE = kTopPSegCap / kThreads;  // entries per thread
  double rem;
  bool use_q;
  const int c = pick_list_chunk(dm, ws, uni, b, resid, rem, use_q);
  // the segment's entries, in registers: index relative to the chunk's first slot, weight
  const size_t seg = (size_t)(b * (K + 1) + n) * dm.nchunks + c;
  const int cnt = min(ws.tkcnt[seg], kTopPSegCap);
  const uint32_t* list = ws.tkept + seg * kTopPSegCap;
  const E* trow = row_ptr(dm, tgt, drf, target_row(dm, b, n));
  const int base = c * dm.chunk_elems - row_phase(trow);  // element index of the chunk's first slot
  const E* drow = resid ? row_ptr(dm, tgt, drf, draft_row(dm, b, n)) : nullptr;
  int ri[PE];
  unsigned long long xw[PE];
#pragma unroll
  for (int i = 0; i < PE; ++i) {
    const int e = tid + kThreads * i;
    ri[i] = -1;
    xw[i] = 0ull;
    if (e < cnt) {
      const int idx = (int)list[e];
      unsigned long long wq, ww;
      list_weights<E>(idx, rt, rd, resid, trow, drow, sp.inv_t, wq, ww);
      ri[i] = idx - base;
      xw[i] = use_q ? wq : ww;
    }
  }
  const int a = pick_in_chunk(rem, [&](int, auto&& add) {
#pragma unroll
    for (int i = 0; i < PE; ++i)
      if (xw[i]) add(ri[i], xw[i]);
  });
  if (tid == 0) {
    out_tokens[(size_t)b * (K + 1) + n] = base + a;
    if (resid && use_q) {  // the residual had zero mass: q is used (reported)
      SeqState s2 = st;
      s2.fallback = 1;
      ws.seq[b] = s2;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Final draw over the edge codes of an fp32 top-p target row (the kept set found from its codes,
// q and p gathered at its indices only).  A thread holds 64 codes of the chunk, bytes
// 16 (t + 256 i) .. + 15 for i < 4; bit 16 i + j of its hit mask is byte j of vector i, which is
// slot 16 t + 4096 i + j of the chunk.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int coded_slot(int k) {
  return 16 * (int)threadIdx.x + 4096 * (k >> 4) + (k & 15);
}

// This thread's 64 codes of chunk c of row r.
__device__ __forceinline__ void coded_load(const Dims& dm, const Workspace& ws, int r, int c,
                                           uint32_t (&w)[16]) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      ws.codes + ((size_t)r * dm.nchunks + c) * dm.chunk_elems, (short)0, dm.chunk_elems,
      0x00020000);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)threadIdx.x * 16, i * kThreads * 16,
                                                       0);
    w[4 * i + 0] = x.x;
    w[4 * i + 1] = x.y;
    w[4 * i + 2] = x.z;
    w[4 * i + 3] = x.w;
  }
}

// Hit mask of this thread's codes: the slots whose code is at most gk.
__device__ __forceinline__ unsigned long long coded_hits(const uint32_t (&w)[16], int gk) {
  unsigned long long mask = 0ull;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
      if ((int)((w[j] >> (8 * bb)) & 0xFFu) <= gk) mask |= 1ull << (4 * j + bb);
  return mask;
}

// Calls f(slot, wq, ww) for every hit of the mask, with the weights of list_weights; the
// logits of up to eight hits (both rows) are loaded together, before any of them is used.  dmask
// (same bit layout): the slots where the draft row may keep its token; elsewhere p = 0 and the
// draft logit is not loaded.
template <class F>
__device__ __forceinline__ void coded_weights(unsigned long long mask, unsigned long long dmask,
                                              int base, const RowStat& rt, const RowStat& rd,
                                              bool resid, const float* __restrict__ trow,
                                              const float* __restrict__ drow, float it, F&& f) {
  constexpr int NB = 8;
  while (mask) {
    int a[NB];
    bool dk[NB];
    float zt[NB], zd[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      a[k] = -1;
      dk[k] = false;
      if (mask) {
        const int kb = __ffsll((long long)mask) - 1;
        a[k] = coded_slot(kb);
        dk[k] = resid && ((dmask >> kb) & 1ull);
        mask &= mask - 1ull;
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      zt[k] = a[k] >= 0 ? trow[base + a[k]] : 0.0f;
      zd[k] = dk[k] ? drow[base + a[k]] : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (a[k] >= 0) {
        unsigned long long wq, ww;
        list_weights_z(zt[k], zd[k], rt, rd, resid, it, wq, ww);
        f(a[k], wq, ww);
      }
    }
  }
}

// The slots of chunk c of draft row n of sequence b where the draft may keep its token (code at
// most the draft threshold's; every slot when the draft row's frame is not the target row's,
// or when the row is not a residual draw).
__device__ __forceinline__ unsigned long long draft_kept_mask(const Dims& dm, const Samp& sp,
                                                              const Workspace& ws, int b, int n,
                                                              int c, const RowStat& rd,
                                                              const float* trow,
                                                              const float* drow) {
  if (drow == nullptr || row_phase(trow) != row_phase(drow)) return ~0ull;
  const int r = draft_row(dm, b, n);
  uint32_t w[16];
  coded_load(dm, ws, r, c, w);
  const ChunkPart part = ws.parts[(size_t)r * dm.nchunks + c];
  const int gk = part.vmax > -INFINITY ? part.pad[0] - topp_edge(rd.thr, sp.inv_t) : -1;
  // (a threshold beyond the codes' reach, gk >= kCodeFar, keeps every slot, far codes too)
  return coded_hits(w, gk);
}

// The chunk's masses of the final weights, as final_lpart, from the codes.
__device__ void final_cpart(const float* __restrict__ tgt, const float* __restrict__ drf,
                            const Dims& dm, const Samp& sp, const Workspace& ws, int b, int c,
                            const SeqState& st, const RowStat& rt, const RowStat& rd) {
  const int n = st.n;
  const bool resid = n < dm.K;
  const int r = target_row(dm, b, n);
  const float* trow = row_ptr(dm, tgt, drf, r);
  const float* drow = resid ? row_ptr(dm, tgt, drf, draft_row(dm, b, n)) : nullptr;
  uint32_t w[16];
  coded_load(dm, ws, r, c, w);  // issued with the chunk's partial: both depend on n only
  const ChunkPart part = ws.parts[(size_t)r * dm.nchunks + c];
  const unsigned long long dmask = draft_kept_mask(dm, sp, ws, b, n, c, rd, trow, drow);
  // kept elements have an edge at or above the threshold's: code <= etop - edge(thr)
  const int gk = part.vmax > -INFINITY ? part.pad[0] - topp_edge(rt.thr, sp.inv_t) : -1;
  const unsigned long long mask = coded_hits(w, gk);
  const int base = c * dm.chunk_elems - row_phase(trow);
  unsigned long long W = 0, Q = 0;
  coded_weights(mask, dmask, base, rt, rd, resid, trow, drow, sp.inv_t,
                [&](int, unsigned long long wq, unsigned long long ww) {
                  W += ww;
                  Q += wq;
                });
  auto add = [](unsigned long long x, unsigned long long y) { return x + y; };
  W = wave_reduce(W, add);
  Q = wave_reduce(Q, add);
  __shared__ unsigned long long s_wq[2][kThreads / 64];
  if (lane_id() == 0) {
    s_wq[0][wave_id()] = W;
    s_wq[1][wave_id()] = Q;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    ws.lpart[(size_t)b * dm.nchunks + c] =
        make_ulonglong2(s_wq[0][0] + s_wq[0][1] + s_wq[0][2] + s_wq[0][3],
                        s_wq[1][0] + s_wq[1][1] + s_wq[1][2] + s_wq[1][3]);
}

// The draw, as final_lpick, from the codes: the chunk from the masses of final_cpart, the
// position inside it from the chunk's hits (pass 1 only rescans the 16 threads whose slots lie
// in bin d1).
__device__ void final_cpick(const float* __restrict__ tgt, const float* __restrict__ drf,
                            const Dims& dm, const Samp& sp, const Workspace& ws,
                            const float* __restrict__ uni, int32_t* __restrict__ out_tokens, int b,
                            const SeqState& st, const RowStat& rt, const RowStat& rd) {
  const int K = dm.K, n = st.n;
  const bool resid = n < K;
  double rem;
  bool use_q;
  const int c = pick_list_chunk(dm, ws, uni, b, resid, rem, use_q);
  const int r = target_row(dm, b, n);
  const float* trow = row_ptr(dm, tgt, drf, r);
  const float* drow = resid ? row_ptr(dm, tgt, drf, draft_row(dm, b, n)) : nullptr;
  uint32_t w[16];
  coded_load(dm, ws, r, c, w);
  const ChunkPart part = ws.parts[(size_t)r * dm.nchunks + c];
  const unsigned long long dmask = draft_kept_mask(dm, sp, ws, b, n, c, rd, trow, drow);
  const int gk = part.vmax > -INFINITY ? part.pad[0] - topp_edge(rt.thr, sp.inv_t) : -1;
  const unsigned long long mask = coded_hits(w, gk);
  const int base = c * dm.chunk_elems - row_phase(trow);
  const float it = sp.inv_t;
  // this thread's first eight hits and their weights, computed once for both passes (both
  // logits of each loaded together); a thread with more hits (rare) recomputes the rest per pass
  constexpr int NH = 8;
  int hs[NH];
  unsigned long long hw[NH];
  unsigned long long rest = mask;
  {
    bool dk[NH];
    float zt[NH], zd[NH];
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      hs[k] = -1;
      dk[k] = false;
      if (rest) {
        const int kb = __ffsll((long long)rest) - 1;
        hs[k] = coded_slot(kb);
        dk[k] = resid && ((dmask >> kb) & 1ull);
        rest &= rest - 1ull;
      }
    }
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      zt[k] = hs[k] >= 0 ? trow[base + hs[k]] : 0.0f;
      zd[k] = dk[k] ? drow[base + hs[k]] : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      hw[k] = 0ull;
      if (hs[k] >= 0) {
        unsigned long long wq, ww;
        list_weights_z(zt[k], zd[k], rt, rd, resid, it, wq, ww);
        hw[k] = use_q ? wq : ww;
      }
    }
  }
  const int a = pick_in_chunk(rem, [&](int d1, auto&& add) {
#pragma unroll
    for (int k = 0; k < NH; ++k)
      if (hs[k] >= 0) add(hs[k], hw[k]);  // (the second pass keeps bin d1's)
    unsigned long long m = rest;
    if (m && d1 >= 0) {  // bin d1: slots 256 d1 .. + 255, vector d1 / 16 of threads 16 (d1 % 16) ..
      const bool mine = ((int)threadIdx.x >> 4) == (d1 & 15);
      m = mine ? (m >> (16 * (d1 >> 4))) & 0xFFFFull : 0ull;
      m <<= 16 * (d1 >> 4);
    }
    coded_weights(m, dmask, base, rt, rd, resid, trow, drow, it,
                  [&](int s, unsigned long long wq, unsigned long long ww) {
                    add(s, use_q ? wq : ww);
                  });
  });
  if (threadIdx.x == 0) {
    out_tokens[(size_t)b * (K + 1) + n] = base + a;
    if (resid && use_q) {  // the residual had zero mass: q is used (reported)
      SeqState s2 = st;
      s2.fallback = 1;
      ws.seq[b] = s2;
    }
  }
}

// ------------------------------------------------------------------------------------------
// k_final_partial: grid = B x final chunks; mass of the final weights per chunk (residual,
// target).  A final chunk is FR vector rows of 256 threads x 16 bytes (FR = kVecPerThread: a
// whole chunk; FR = 4 or 1 when the sequences are fewer and each chunk is split).
// ------------------------------------------------------------------------------------------
template <class E, bool VEC, int FR, bool LIST>
__global__ __launch_bounds__(kThreads) void k_final_partial(const E* __restrict__ tgt,
                                                            const E* __restrict__ drf, Dims dm,
                                                            Samp sp, Workspace ws) {
  // LIST (top-p): max(final chunks, chunks) workgroups per sequence; a sequence drawn from its
  // kept segments takes the first `chunks` of them, one per segment
  // (LIST: chunk-major, blockIdx = c B + b, so that the workgroups of the kept-list draws,
  // c < chunks, are dispatched first and spread over the XCDs)
  const int G = LIST ? max(dm.nfchunks, dm.nchunks) : dm.nfchunks;
  const int bid = LIST ? (int)blockIdx.x : xcd_contiguous((int)blockIdx.x, dm.B * G);
  const int b = LIST ? bid % dm.B : bid / G;
  const int c = LIST ? bid / dm.B : bid - (bid / G) * G;
  // the state and the rows' statistics in one step (the statistics are stale, and unused,
  // when the sequence needs no draw here)
  const SeqState st = ws.seq[b];
  const RowStat rt = ws.dstat[2 * b], rd = ws.dstat[2 * b + 1];
  if constexpr (LIST) {
    if (st.need_list) {
      if (c < dm.nchunks) {
        if constexpr (sizeof(E) == 4)
          final_cpart(tgt, drf, dm, sp, ws, b, c, st, rt, rd);
        else
          final_lpart<E>(tgt, drf, dm, sp, ws, b, c, st, rt, rd);
      }
      return;
    }
  }
  if (!st.need_dense || c >= dm.nfchunks) return;
  __shared__ RedScratch red;
  const int n = st.n;
  const DrawRows g = draw_rows(dm, n, rt, rd);
  const E* trow = row_ptr(dm, tgt, drf, target_row(dm, b, n));
  const E* drow = g.resid ? row_ptr(dm, tgt, drf, draft_row(dm, b, n)) : trow;
  const int c0 = c * dm.fchunk_elems;
  const int cend = min(c0 + dm.fchunk_elems, dm.V);
  const float it = sp.inv_t;
  constexpr int EPV = Tr<E>::kEpv;
  // steps of NV vectors per thread of both rows; the next step's loads are issued before a
  // step is summed
  constexpr int NV0 = EPV == 8 ? 2 : 4;
  constexpr int NV = NV0 < FR ? NV0 : FR;
  constexpr int NS = FR / NV;
  constexpr int STEP = kThreads * NV * EPV;
  double W = 0.0, Q = 0.0;
  auto sum_step = [&](const uint32_t(&xt)[4 * NV], const uint32_t(&xd)[4 * NV], int s) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float wv = 0.0f, qv = 0.0f;
      const int e = c0 + s * STEP + ((int)threadIdx.x + kThreads * i) * EPV;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int h = 0; h < Tr<E>::kPerDword; ++h) {
          float w, q;
          draw_weights(e < cend ? Tr<E>::elem(xt[4 * i + d], h) : -INFINITY,
                       g.resid ? Tr<E>::elem(xd[4 * i + d], h) : 0.0f, g, it, w, q);
          wv += w;
          qv += q;
        }
      }
      W += (double)wv;
      Q += (double)qv;
    }
  };
  uint32_t at[4 * NV], ad[4 * NV], bt[4 * NV], bd[4 * NV];
  load_vecs<E, VEC, NV, true>(trow, cend, c0, at);
  if (g.resid) load_vecs<E, VEC, NV, true>(drow, cend, c0, ad);
  if constexpr (NS == 1) sum_step(at, ad, 0);
#pragma unroll 1
  for (int s = 0; NS > 1 && s < NS; s += 2) {
    load_vecs<E, VEC, NV, true>(trow, cend, c0 + (s + 1) * STEP, bt);
    if (g.resid) load_vecs<E, VEC, NV, true>(drow, cend, c0 + (s + 1) * STEP, bd);
    sum_step(at, ad, s);
    // past the chunk's last step this loads nothing: the buffer range check covers it
    load_vecs<E, VEC, NV, true>(trow, cend, c0 + (s + 2) * STEP, at);
    if (g.resid) load_vecs<E, VEC, NV, true>(drow, cend, c0 + (s + 2) * STEP, ad);
    sum_step(bt, bd, s + 1);
  }
  W = block_sum_d(W, red);
  Q = block_sum_d(Q, red);
  if (threadIdx.x == 0) ws.fpart[(size_t)b * dm.nfchunks + c] = make_double2(W, Q);
}

// Exclusive prefix of one double per thread over the workgroup, in thread order (fixed order:
// a scan inside each wave, then the wave totals in order).  Also returns the total.
__device__ double block_exclusive_d(double v, double& total, RedScratch& red) {
  double x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane_id() >= o) x += y;
  }
  __syncthreads();
  if (lane_id() == 63) red.d[wave_id()] = x;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave_id(); ++w) base += red.d[w];
  total = ((red.d[0] + red.d[1]) + red.d[2]) + red.d[3];
  return base + (x - v);
}

// The same for two doubles per thread at once (one set of shuffles and barriers): returns the
// exclusive prefix of a and sets b_ex, and the totals.
__device__ double block_exclusive_d2(double a, double b, double& a_tot, double& b_tot,
                                     double& b_ex) {
  __shared__ double s_w[2][kThreads / 64];
  double x = a, y = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double xs = __shfl_up(x, o), ys = __shfl_up(y, o);
    if (lane_id() >= o) {
      x += xs;
      y += ys;
    }
  }
  __syncthreads();
  if (lane_id() == 63) {
    s_w[0][wave_id()] = x;
    s_w[1][wave_id()] = y;
  }
  __syncthreads();
  double ba = 0.0, bb = 0.0;
  for (int w = 0; w < wave_id(); ++w) {
    ba += s_w[0][w];
    bb += s_w[1][w];
  }
  a_tot = ((s_w[0][0] + s_w[0][1]) + s_w[0][2]) + s_w[0][3];
  b_tot = ((s_w[1][0] + s_w[1][1]) + s_w[1][2]) + s_w[1][3];
  b_ex = bb + (y - b);
  return ba + (x - a);
}

// ------------------------------------------------------------------------------------------
// k_small: problems whose every sequence fits one workgroup's registers (2K+1 rows of V logits,
// at most kSmallRegs per thread), dense rows only (T > 0, nothing truncated): one workgroup per
// sequence reads its rows once and does the row statistics, the accept scan and the final
// draw in a single launch (the multi-kernel path needs four launches, which dominate at such
// sizes).  Thread t holds elements [t L, t L + L) of every row (-inf past V); the final draw
// takes the first thread whose range of the running weight passes u W (weights as in the
// chunked draw: fp32 per element with reciprocal normalisers, fp64 across), then the element
// inside it; past the end (rounding), the last element with weight.
// ------------------------------------------------------------------------------------------
constexpr int kSmallRegs = 64;

template <class E, int L>
__global__ __launch_bounds__(kThreads) void k_small(const E* __restrict__ tgt,
                                                    const E* __restrict__ drf, Dims dm, Samp sp,
                                                    Workspace ws, Outs o) {
  constexpr int RMAX = kSmallRegs / L;
  constexpr int SH = 6 - log2_pow2(RMAX);  // row r's wave total is in lanes r << SH, ...
  const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int K = dm.K, R = dm.rows_per_seq;  // rows: target 0..K, then draft 0..K-1
  const float it = sp.inv_t;
  __shared__ float s_m[RMAX][kThreads / 64];
  __shared__ double s_s[RMAX][kThreads / 64];
  __shared__ RowStat s_rs[RMAX];
  __shared__ int s_n;
  __shared__ RedScratch red;
  const int e0 = tid * L;
  __shared__ int s_x[RMAX];           // draft tokens
  __shared__ float s_zx[RMAX][2];     // target and draft logits at them
  if (tid < K) s_x[tid] = o.drafts[(size_t)b * K + tid];
  float z[RMAX][L];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const E* row = row_ptr(dm, tgt, drf, b * R + (r < R ? r : 0));
#pragma unroll
    for (int e = 0; e < L; ++e)
      z[r][e] = (r < R && e0 + e < dm.V) ? load_logit(row, e0 + e) : -INFINITY;
  }
  // row maxima, then normalisers: fp32 over a thread's elements, fp64 across (fixed orders; the
  // rows of a wave reduced together by recursive halving; rows past R hold -inf: they are
  // reduced too, and never read)
  {
    float mx[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      mx[r] = -INFINITY;
#pragma unroll
      for (int e = 0; e < L; ++e) mx[r] = fmaxf(mx[r], z[r][e]);
    }
    const float t = wave_reduce_halving(mx, [](float x, float y) { return fmaxf(x, y); });
    if ((lane & ((1 << SH) - 1)) == 0) s_m[lane >> SH][wv] = t;
  }
  __syncthreads();
  // the logits at the draft tokens, from the thread holding them: row r is target row r
  // (r <= K) or draft row r - K - 1, either read at draft token k of its position
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const bool is_t = r <= K;
    const int k = is_t ? r : r - K - 1;
    const int x = r < R && k < K ? s_x[k] : -1;
    if (x >= 0 && x < dm.V && x / L == tid) {
      float v = 0.0f;
#pragma unroll
      for (int j = 0; j < L; ++j)
        if (e0 + j == x) v = z[r][j];
      s_zx[k][is_t ? 0 : 1] = v;
    }
  }
  {
    double sd[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      const float m = fmaxf(fmaxf(s_m[r][0], s_m[r][1]), fmaxf(s_m[r][2], s_m[r][3]));
      float sv = 0.0f;
      if (r < R) {
#pragma unroll
        for (int e = 0; e < L; ++e) sv += fast_exp((z[r][e] - m) * it);
      }
      sd[r] = (double)sv;
    }
    const double t = wave_reduce_halving(sd, [](double x, double y) { return x + y; });
    if ((lane & ((1 << SH) - 1)) == 0) s_s[lane >> SH][wv] = t;
  }
  __syncthreads();
  if (tid < R) {
    RowStat rs;
    rs.m = fmaxf(fmaxf(s_m[tid][0], s_m[tid][1]), fmaxf(s_m[tid][2], s_m[tid][3]));
    rs.thr = -INFINITY;
    rs.S = ((s_s[tid][0] + s_s[tid][1]) + s_s[tid][2]) + s_s[tid][3];
    rs.argmax = -1;
    rs.nkept = -1;
    rs.kind = kRowDense;
    rs.pad = 0;
    s_rs[tid] = rs;
  }
  __syncthreads();
  if (wv == 0) {
    const int base = b * R;
    const int n = seq_accept_wave(
        tgt, drf, dm, sp, ws, o, b, [&](int r) { return s_rs[r - base]; },
        [&](int k, int, float& zt, float& zd) {
          zt = s_zx[k][0];
          zd = s_zx[k][1];
        },
        lane < K ? s_x[lane] : -2);
    if (lane == 0) s_n = n;
  }
  __syncthreads();
  const int n = s_n;
  const bool resid = n < K;
  const DrawRows g = draw_rows(dm, n, s_rs[n], s_rs[resid ? K + 1 + n : n]);
  // the final pair's weights, its rows taken from the registers by predicated moves
  float wq[L], ww[L];
#pragma unroll
  for (int e = 0; e < L; ++e) {
    float zt = -INFINITY, zd = -INFINITY;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r == n) zt = z[r][e];
      if (resid && r == K + 1 + n) zd = z[r][e];
    }
    draw_weights(zt, zd, g, it, ww[e], wq[e]);
  }
  double wl = 0.0, ql = 0.0;  // this thread's masses, in index order
#pragma unroll
  for (int e = 0; e < L; ++e) {
    wl += (double)ww[e];
    ql += (double)wq[e];
  }
  double Wt, Qt, qex;
  const double wex = block_exclusive_d2(wl, ql, Wt, Qt, qex);
  const bool use_q = !resid || !(Wt > 0.0);
  const double ex = use_q ? qex : wex, loc = use_q ? ql : wl;
  const double target = (double)o.uni[(size_t)b * (K + 1) + K] * (use_q ? Qt : Wt);
  // the first thread whose range passes the target, else the last thread with mass
  const int th = block_min_i(loc > 0.0 && ex + loc > target ? tid : INT_MAX, red);
  const int tl = block_max_i(loc > 0.0 ? tid : -1, red);
  const int owner = th != INT_MAX ? th : tl;
  if (tid == owner) {
    const double rem = target - ex;
    double cum = 0.0;
    int pick = -1, last = 0;
#pragma unroll
    for (int e = 0; e < L; ++e) {
      const double v = (double)(use_q ? wq[e] : ww[e]);
      if (v > 0.0) {
        last = e;
        cum += v;
        if (pick < 0 && th != INT_MAX && cum > rem) pick = e;
      }
    }
    o.tokens[(size_t)b * (K + 1) + n] = e0 + (pick >= 0 ? pick : last);
  }
}


// ------------------------------------------------------------------------------------------
// k_final_pick: grid = B.  Chooses the final chunk holding u*W from the chunk totals (scanned
// in order), then the token inside it in three steps, all in index order: the chunk is loaded
// as a register tile of NR vector rows (thread t, vector i covers elements
// c0 + (t + 256 i) * EPV ...), so vector row i (all threads' vector i) precedes row i + 1; the
// row sums locate the vector row, a workgroup scan over the row's vectors locates the vector,
// and its owner finds the index.  With a single chunk the chunk pass is skipped and the totals
// come from the tile itself.
// ------------------------------------------------------------------------------------------
template <class E, bool VEC, int NR, bool LIST>
__global__ __launch_bounds__(kThreads) void k_final_pick(const E* __restrict__ tgt,
                                                         const E* __restrict__ drf, Dims dm,
                                                         Samp sp, Workspace ws,
                                                         const float* __restrict__ uni,
                                                         int32_t* __restrict__ out_tokens) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  constexpr int EPV = Tr<E>::kEpv;
  const int K = dm.K;
  const bool single = dm.nfchunks == 1;
  // chunk totals: thread t owns chunks [t * per, (t + 1) * per)
  const double2* fp = ws.fpart + (size_t)b * dm.nfchunks;
  const int per = (dm.nfchunks + kThreads - 1) / kThreads;
  const int ca = min(dm.nfchunks, tid * per), cb = min(dm.nfchunks, ca + per);
  // the state, the rows' statistics, the uniform and the chunk totals in one step (all but
  // the state are stale, and unused, when the sequence needs no dense draw)
  const SeqState st = ws.seq[b];
  const RowStat srt = ws.dstat[2 * b], srd = ws.dstat[2 * b + 1];
  const double u = (double)uni[(size_t)b * (K + 1) + K];
  // a thread's first chunk stays in registers (with at most 256 chunks, its only one)
  const double2 first = !single && ca < cb ? fp[ca] : make_double2(0.0, 0.0);
  auto mass = [&](int cc, bool q) {
    const double2 m = cc == ca ? first : fp[cc];
    return q ? m.y : m.x;
  };
  double w_loc = 0.0, q_loc = 0.0;
  if (!single) {
    for (int cc = ca; cc < cb; ++cc) {
      w_loc += mass(cc, false);
      q_loc += mass(cc, true);
    }
  }
  if constexpr (LIST) {
    if (st.need_list) {  // top-p: the draw from the kept segments (bf16) or the codes (fp32)
      if constexpr (sizeof(E) == 4)
        final_cpick(tgt, drf, dm, sp, ws, uni, out_tokens, b, st, srt, srd);
      else
        final_lpick<E>(tgt, drf, dm, sp, ws, uni, out_tokens, b, st, srt, srd);
      return;
    }
  }
  if (!st.need_dense) return;
  __shared__ RedScratch red;
  __shared__ float s_vw[NR][kThreads], s_vq[NR][kThreads];  // per-vector sums
  __shared__ double s_rw[NR], s_rq[NR];                       // per-row sums
  __shared__ int s_chunk, s_last, s_t, s_tl;
  __shared__ double s_before;
  const int n = st.n;
  const DrawRows g = draw_rows(dm, n, srt, srd);
  bool use_q = !g.resid;
  double target = 0.0;
  int c = 0;
  if (!single) {
    double Wt, Qt;
    double q_ex;
    double w_ex = block_exclusive_d2(w_loc, q_loc, Wt, Qt, q_ex);
    use_q = !(Wt > 0.0) || !g.resid;
    if (use_q) w_ex = q_ex;
    target = u * (use_q ? Qt : Wt);
    if (tid == 0) {
      s_chunk = INT_MAX;
      s_last = -1;
    }
    __syncthreads();
    double cum = w_ex;
    int found = INT_MAX, lastc = -1;
    for (int cc = ca; cc < cb; ++cc) {
      const double v = mass(cc, use_q);
      if (v > 0.0) lastc = cc;
      if (found == INT_MAX && cum + v > target) found = cc;
      cum += v;
    }
    if (found != INT_MAX) atomicMin(&s_chunk, found);
    if (lastc >= 0) atomicMax(&s_last, lastc);
    __syncthreads();
    c = s_chunk != INT_MAX ? s_chunk : s_last;
    if (c >= ca && c < cb) {  // the owner of chunk c: the mass before it, as summed above
      double cb4 = w_ex;
      for (int cc = ca; cc < c; ++cc) cb4 += mass(cc, use_q);
      s_before = cb4;
    }
  }
  const E* trow = row_ptr(dm, tgt, drf, target_row(dm, b, n));
  const E* drow = g.resid ? row_ptr(dm, tgt, drf, draft_row(dm, b, n)) : trow;
  const int c0 = c * dm.fchunk_elems;
  const int cend = min(c0 + dm.fchunk_elems, dm.V);
  const float it = sp.inv_t;
  // per-vector sums of the chunk
  constexpr int NV = NR < 4 ? NR : 4;
  uint32_t rt[4 * NV], rd[4 * NV];  // with NR <= 4 the whole tile, kept for the last step
#pragma unroll 1
  for (int s = 0; s < NR / NV; ++s) {
    const int base = c0 + s * kThreads * NV * EPV;
    load_vecs<E, VEC, NV, true>(trow, cend, base, rt);
    if (g.resid) load_vecs<E, VEC, NV, true>(drow, cend, base, rd);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = base + (tid + kThreads * i) * EPV;
      float wv = 0.0f, qv = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int h = 0; h < Tr<E>::kPerDword; ++h) {
          float w, q;
          draw_weights(e < cend ? Tr<E>::elem(rt[4 * i + d], h) : -INFINITY,
                       g.resid ? Tr<E>::elem(rd[4 * i + d], h) : 0.0f, g, it, w, q);
          wv += w;
          qv += q;
        }
      }
      s_vw[s * NV + i][tid] = wv;
      s_vq[s * NV + i][tid] = qv;
    }
  }
  __syncthreads();
  // row sums: wave w takes rows w, w + 4, ... (fixed order inside each row)
  for (int i = wv; i < NR; i += 4) {
    double sw = 0.0, sq = 0.0;
#pragma unroll
    for (int j = 0; j < kThreads / 64; ++j) {
      sw += (double)s_vw[i][lane * (kThreads / 64) + j];
      sq += (double)s_vq[i][lane * (kThreads / 64) + j];
    }
    sw = wave_reduce(sw, [](double x, double y) { return x + y; });
    sq = wave_reduce(sq, [](double x, double y) { return x + y; });
    if (lane == 0) {
      s_rw[i] = sw;
      s_rq[i] = sq;
    }
  }
  __syncthreads();
  double before = 0.0;
  if (single) {
    double Wt = 0.0, Qt = 0.0;
    for (int i = 0; i < NR; ++i) {
      Wt += s_rw[i];
      Qt += s_rq[i];
    }
    use_q = !(Wt > 0.0) || !g.resid;
    target = u * (use_q ? Qt : Wt);
  } else {
    before = s_before;
  }
  if (tid == 0 && g.resid && use_q) {  // the residual had zero mass: q is used (reported)
    SeqState s2 = st;
    s2.fallback = 1;
    ws.seq[b] = s2;
  }
  const float(*sv)[kThreads] = use_q ? s_vq : s_vw;
  const double* rs = use_q ? s_rq : s_rw;
  // the vector row
  int ri = -1, rlast = -1;
  double cum = before, cum_last = before;
  for (int i = 0; i < NR; ++i) {
    if (rs[i] > 0.0) {
      rlast = i;
      cum_last = cum;
    }
    if (ri < 0 && cum + rs[i] > target) {
      ri = i;
      break;
    }
    cum += rs[i];
  }
  const bool clamp = ri < 0;  // rounding left u*W at or past the total: the last positive
  if (clamp) {
    ri = rlast < 0 ? 0 : rlast;
    cum = cum_last;
  }
  // the vector inside row ri
  const double v = (double)sv[ri][tid];
  double rtot;
  const double vex = block_exclusive_d(v, rtot, red);
  if (tid == 0) {
    s_t = INT_MAX;
    s_tl = -1;
  }
  __syncthreads();
  // the last positive vector and the first one past the target: one LDS atomic per wave
  const unsigned long long pos = __ballot(v > 0.0);
  const unsigned long long hit = __ballot(v > 0.0 && !clamp && cum + vex + v > target);
  if (lane == 0) {
    if (pos) atomicMax(&s_tl, wv * 64 + 63 - __clzll((long long)pos));
    if (hit) atomicMin(&s_t, wv * 64 + __ffsll((long long)hit) - 1);
  }
  __syncthreads();
  int tt = s_t;
  const bool last = clamp || tt == INT_MAX;  // fall back to the last positive vector
  if (last) tt = s_tl;
  if (tid == (tt < 0 ? 0 : tt)) {
    int pick = -1;
    if (tt >= 0) {
      const int e = c0 + (tt + kThreads * ri) * EPV;
      float zt[EPV], zd[EPV];
      if constexpr (NR == NV) {  // this thread's vector ri of the tile, as summed above
        uint32_t wt[4], wd[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          wt[d] = rt[d];
          wd[d] = rd[d];
        }
#pragma unroll
        for (int i = 1; i < NV; ++i) {
          if (ri == i) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              wt[d] = rt[4 * i + d];
              wd[d] = rd[4 * i + d];
            }
          }
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int h = 0; h < Tr<E>::kPerDword; ++h) {
            zt[d * Tr<E>::kPerDword + h] = e < cend ? Tr<E>::elem(wt[d], h) : -INFINITY;
            zd[d * Tr<E>::kPerDword + h] = g.resid ? Tr<E>::elem(wd[d], h) : 0.0f;
          }
        }
      } else {
        load_vec_f<E, VEC>(trow, cend, e, zt);
        if (g.resid) load_vec_f<E, VEC>(drow, cend, e, zd);
      }
      double run = cum + vex;
      int lastpos = -1;
#pragma unroll
      for (int x = 0; x < EPV; ++x) {
        float w, q;
        draw_weights(zt[x], g.resid ? zd[x] : 0.0f, g, it, w, q);
        const float wx = use_q ? q : w;
        if (wx > 0.0f) lastpos = e + x;
        run += (double)wx;
        if (!last && pick < 0 && wx > 0.0f && run > target) pick = e + x;
      }
      if (pick < 0) pick = lastpos;
    }
    if (pick < 0) pick = c0;  // no positive weight in the chunk (cannot happen for a valid row)
    out_tokens[(size_t)b * (K + 1) + n] = pick;
  }
}

// ------------------------------------------------------------------------------------------
// Compact top-k path, two launches and no communication between workgroups inside a launch
// (on this GPU an agent-scope release per workgroup, needed to publish partial results to
// another workgroup, costs far more than the streaming itself).
//   k_topk_row : one workgroup per row streams the row in register tiles and keeps, per wave,
//                a list of candidates (every element >= a threshold that never exceeds the
//                row's k-th largest); at the end one wave selects the row's k-th largest among
//                them (the row's top-k set, ties included, is among the candidates) and writes
//                (m, thr, S) and the kept tokens.
//   k_seq_compact : one workgroup per sequence: accept tests, first rejection, final draw.
// ------------------------------------------------------------------------------------------
constexpr int kWaveListCap = 512;  // candidates one wave may hold for a row

// Order-preserving barrier between lanes of one wave communicating through LDS.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}


struct alignas(16) RowLds {
  // per-wave candidate lists: canonical keys and vocabulary indices; entries kWaveListCap ..
  // kWaveListCap + 63 are per-lane sinks for the stores of lanes without a candidate
  uint32_t key[4][kWaveListCap + 64];
  uint32_t idx[4][kWaveListCap + 64];
  RedScratch red;
  uint32_t tmax[kThreads];        // per-thread maxima of tile 0
  uint32_t tau;
  uint32_t wtau[4];               // each wave's latest filter threshold, read by the others
  uint32_t ckey[kKeptCap];        // the row's top-k set, compacted by the merge (keys) ...
  uint32_t cidx[kKeptCap];        // ... and vocabulary indices
  int cnt[4];
  int ovf[4];
  int fallback;
};

// One wave's candidate list (row w of RowLds); every field has the same value in all lanes.
struct WaveList {
  int w;
  int count;
  int ovf;
  uint32_t tau;  // filter threshold on (non-canonical) keys
};

// Appends up to two entries per lane (h0: (i0, k0), h1: (i1, k1)) in (lane, half) order, with
// no branch: a lane without an entry stores to its sink slot.
__device__ __forceinline__ void wl_push(RowLds& S, WaveList& L, bool h0, uint32_t i0, uint32_t k0,
                                        bool h1, uint32_t i1, uint32_t k1) {
  const unsigned long long m0 = __ballot(h0), m1 = __ballot(h1);
  const unsigned long long below = lanes_below();
  const int pos = L.count + __popcll(m0 & below) + __popcll(m1 & below);
  const int sink = kWaveListCap + lane_id();
  const int p0 = (h0 && pos < kWaveListCap) ? pos : sink;
  const int p1 = (h1 && pos + (int)h0 < kWaveListCap) ? pos + (int)h0 : sink;
  S.key[L.w][p0] = k0;
  S.idx[L.w][p0] = i0;
  S.key[L.w][p1] = k1;
  S.idx[L.w][p1] = i1;
  L.count += __popcll(m0) + __popcll(m1);
}

// Threshold on non-canonical keys equivalent to "value >= value of canonical key x".
template <class E>
__device__ __forceinline__ uint32_t filter_tau(uint32_t x) {
  if (x < 1u) x = 1u;                                 // key 0 marks slots past the row end
  return x == Tr<E>::kKeyPos0 ? Tr<E>::kKeyNeg0 : x;  // -0 equals +0
}

// Raise the wave's tau to the k-th largest key of its list and drop the entries below it.
// The wave's k-th largest never exceeds the row's, so the row's top-k set stays covered.
template <class E>
__device__ __forceinline__ void wl_raise(RowLds& S, WaveList& L, int k) {
  const int lane = lane_id();
  if (L.count > kWaveListCap) L.ovf = 1;  // entries were lost: the row takes the fallback path
  const int n = L.count < kWaveListCap ? L.count : kWaveListCap;
  wave_lds_sync();
  uint32_t x = 0;
  for (int bit = Tr<E>::kKeyBits - 1; bit >= 0; --bit) {
    const uint32_t cand = x | (1u << bit);
    int c = 0;
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int j = j0 + lane;
      c += __popcll(__ballot(j < n && S.key[L.w][j] >= cand));
    }
    if (c >= k) x = cand;
  }
  int base = 0;
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    const bool keep = j < n && S.key[L.w][j] >= x;
    const uint32_t kk = keep ? S.key[L.w][j] : 0u, ii = keep ? S.idx[L.w][j] : 0u;
    const unsigned long long m = __ballot(keep);
    wave_lds_sync();
    if (keep) {
      const int pos = base + __popcll(m & lanes_below());
      S.key[L.w][pos] = kk;
      S.idx[L.w][pos] = ii;
    }
    base += __popcll(m);
    wave_lds_sync();
  }
  L.count = base;
  const uint32_t t = filter_tau<E>(x);
  if (t > L.tau) L.tau = t;
  // publish it: every wave's threshold is at most the row's k-th largest, so each wave may
  // filter with the largest one published (a stale read is a lower, still valid, bound)
  if (lane == 0) __hip_atomic_store(&S.wtau[L.w], L.tau, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The largest threshold any wave of the row has published, if above the wave's own.
__device__ __forceinline__ void wl_shared_tau(RowLds& S, WaveList& L) {
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    t = max(t, __hip_atomic_load(&S.wtau[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
  t = (uint32_t)__builtin_amdgcn_readfirstlane((int)t);
  if (t > L.tau) L.tau = t;
}

// Per-lane select: lanes in `mask` take hi, the others lo (one v_cndmask_b32).  Written as asm
// so that the compiler cannot fold a tree of these selects back into an indexed load, which
// would move the whole register tile to scratch memory.
__device__ __forceinline__ uint32_t lane_select(unsigned long long mask, uint32_t lo,
                                                uint32_t hi) {
  uint32_t out;
  asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(out) : "v"(lo), "v"(hi), "s"(mask));
  return out;
}

// regs[j] for a per-lane index j in [0, 64): a select tree on the bits of j (m[b] = the lanes
// whose j has bit b set), depth first so that few partial results are live at once.  Every
// lane may ask for a different register without leaving the register file.
template <int N>
__device__ __forceinline__ uint32_t sel_tree(const uint32_t (&r)[kRegs], int base,
                                             const unsigned long long (&m)[6]) {
  if constexpr (N == 1) {
    return r[base];
  } else {
    constexpr int bit = N == 2 ? 0 : N == 4 ? 1 : N == 8 ? 2 : N == 16 ? 3 : N == 32 ? 4 : 5;
    const uint32_t lo = sel_tree<N / 2>(r, base, m);
    const uint32_t hi = sel_tree<N / 2>(r, base + N / 2, m);
    return lane_select(m[bit], lo, hi);
  }
}

__device__ __forceinline__ uint32_t reg_select(const uint32_t (&r)[kRegs], int j) {
  unsigned long long m[6];
#pragma unroll
  for (int b = 0; b < 6; ++b) m[b] = __ballot((j >> b) & 1);
  return sel_tree<kRegs>(r, 0, m);
}

// One register tile of the 16-byte aligned part of a row for the top-k stream: raw buffer loads
// over [c0, c0 + clen) whose range check returns 0 past its end (clen <= 0: nothing is read),
// so no register is rewritten after the loads; the raw path treats such a 0 (+0.0) as below
// every positive tau, and tile_key maps those slots to key 0.
template <class E>
__device__ __forceinline__ void load_tile(const E* __restrict__ row, int c0, int clen,
                                          uint32_t (&regs)[kRegs]) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<E*>(row + c0), (short)0, (clen > 0 ? clen : 0) * (int)sizeof(E), 0x00020000);
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, threadIdx.x * 16, i * kThreads * 16, 2);
    regs[4 * i + 0] = x.x;
    regs[4 * i + 1] = x.y;
    regs[4 * i + 2] = x.z;
    regs[4 * i + 3] = x.w;
  }
}

// Keys of register j of the tile (raw bits in regs); slots past the end of the row get key 0.
// `valid` holds, per vector i, the lanes whose vector i lies inside the row.
template <class E>
__device__ __forceinline__ uint32_t tile_key(const uint32_t (&regs)[kRegs], int j,
                                             const unsigned long long (&valid)[kVecPerThread]) {
  return lane_select(valid[j >> 2], 0u, Tr<E>::keys_of_dword(regs[j]));
}

template <class E>
__device__ __forceinline__ void tile_valid(int clen, unsigned long long (&valid)[kVecPerThread]) {
  const int nvec = clen / Tr<E>::kEpv;  // clen is a multiple of the vector width (or <= 0)
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) valid[i] = __ballot((int)threadIdx.x + kThreads * i < nvec);
}

// Candidates of one tile (raw bits in regs) into the wave's list.  KEYS: compare order-preserving
// keys; otherwise compare raw bits, which is valid only while tau is a positive value (an element is >= tau
// exactly when its bits, read as a signed integer, are >= the bits of tau; slots past the row
// end read as 0, below the bits of any positive tau).  First a per-lane mask of the registers holding a
// candidate, without branches; then one pass per candidate register of the busiest lane, each
// lane taking its lowest remaining register.
template <class E, bool KEYS>
__device__ __forceinline__ void filter_tile(const uint32_t (&regs)[kRegs], int c0,
                                            const unsigned long long (&valid)[kVecPerThread],
                                            RowLds& S, WaveList& L, int k, int raise_at) {
  // Register j has a candidate iff max(w, t) != t with t = tau - 1 (per 16-bit half for bf16;
  // unsigned on keys, signed on raw bits).  The mask bits are shifted in, register j of each
  // half-tile ending at bit 31 - (j mod 32); no compares into VCC and no per-bit constants.
  uint32_t mlo = 0, mhi = 0;
  if constexpr (Tr<E>::kPerDword == 2) {
    typedef short s2 __attribute__((ext_vector_type(2)));
    const uint32_t tm1 = KEYS ? L.tau - 1u : (L.tau & 0x7FFFu) - 1u;
    const uint32_t tpair = tm1 | (tm1 << 16);
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
      uint32_t mx;
      if constexpr (KEYS)
        mx = Tr<E>::dword_max(tile_key<E>(regs, j, valid), tpair);
      else
        mx = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
                                              __builtin_bit_cast(s2, regs[j]),
                                              __builtin_bit_cast(s2, tpair)));
      const uint32_t bit = min(mx ^ tpair, 1u);
      if (j < 32)
        mlo = (mlo << 1) | bit;
      else
        mhi = (mhi << 1) | bit;
    }
  } else {
    const uint32_t tm1 = KEYS ? L.tau - 1u : (L.tau & 0x7FFFFFFFu) - 1u;
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {
      const uint32_t mx =
          KEYS ? max(tile_key<E>(regs, j, valid), tm1) : (uint32_t)max((int)regs[j], (int)tm1);
      const uint32_t bit = min(mx ^ tm1, 1u);
      if (j < 32)
        mlo = (mlo << 1) | bit;
      else
        mhi = (mhi << 1) | bit;
    }
  }
  while (true) {
    const bool has = (mlo | mhi) != 0u;
    if (__ballot(has) == 0ull) break;
    if (L.count > raise_at) wl_raise<E>(S, L, k);
    const int j = mlo ? __builtin_clz(mlo) : (mhi ? 32 + __builtin_clz(mhi) : 0);
    if (mlo)
      mlo &= ~(0x80000000u >> j);
    else
      mhi &= ~(0x80000000u >> (j - 32));
    const uint32_t w = reg_select(regs, j);
    const int i = j >> 2, d = j & 3;
    const uint32_t tau = L.tau;
    if constexpr (Tr<E>::kPerDword == 2) {
      const uint32_t k0 = Tr<E>::key_of_bits(w & 0xFFFFu);
      const uint32_t k1 = Tr<E>::key_of_bits(w >> 16);
      wl_push(S, L, has && k0 >= tau, slot_index<E>(c0, i, d, 0), Tr<E>::canon(k0),
              has && k1 >= tau, slot_index<E>(c0, i, d, 1), Tr<E>::canon(k1));
    } else {
      const uint32_t k0 = Tr<E>::key_of_bits(w);
      wl_push(S, L, has && k0 >= tau, slot_index<E>(c0, i, d, 0), Tr<E>::canon(k0), false, 0u,
              0u);
    }
  }
}

// Top-p on the renormalised top-k set (compacted in S.ckey, nk <= 64 QL entries, all >= x):
// the largest key v such that the entries at or above v carry at least P of the kept mass
// (every entry tied with the boundary is kept), bit by bit from the most significant, each
// lane holding entries lane + 64 i.  Masses are fp64 sums in a fixed order (slots, then the
// wave butterfly), so the result does not change from run to run.  Sets tkey and Ssum (the
// kept set's normaliser).
template <class E, int QL>
__device__ void topp_compact(const Samp& sp, RowLds& S, int nk, float m, double& Ssum,
                             uint32_t& tkey) {
  constexpr int KB = Tr<E>::kKeyBits;
  const int lane = lane_id();
  const float it = sp.inv_t;
  uint32_t kc[QL];
  float ec[QL];
#pragma unroll
  for (int i = 0; i < QL; ++i) {
    const int j = lane + 64 * i;
    kc[i] = j < nk ? S.ckey[j] : 0u;
    ec[i] = j < nk ? fast_exp((Tr<E>::key_to_float(kc[i]) - m) * it) : 0.0f;
  }
  auto mass_ge = [&](uint32_t v) {
    // opaque weights: the conversions are redone per call rather than kept live
#pragma unroll
    for (int i = 0; i < QL; ++i) asm volatile("" : "+v"(ec[i]));
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < QL; ++i)
      if (kc[i] >= v) t += (double)ec[i];
    return wave_reduce(t, [](double a, double b) { return a + b; });
  };
  const uint32_t x = tkey;
  const double need = (double)sp.top_p * Ssum;
  // the result lies in [x, the largest key]: only the bits below their common prefix vary
  uint32_t mk = 0;
#pragma unroll
  for (int i = 0; i < QL; ++i) mk = kc[i] > mk ? kc[i] : mk;
  mk = wave_reduce(mk, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  const int hb = 31 - __builtin_clz((x ^ mk) | 1u);
  uint32_t v = hb == 31 ? 0u : x & ~((2u << hb) - 1u);
  for (int bit = hb; bit >= 0; --bit) {
    const uint32_t cand = v | (1u << bit);
    // every entry is >= x, so mass_ge(cand) = Ssum >= need for cand <= x
    if (cand <= x || mass_ge(cand) >= need) v = cand;
  }
  tkey = v;
  Ssum = mass_ge(tkey);
}

// One wave merges the row from the four wave lists: the row maximum (the largest candidate:
// the maximum is >= every threshold used), the k-th largest key, top-p on the kept set if
// requested; writes RowStat and the kept list (candidate order).  Returns 1, writing nothing,
// when the kept set would not fit kKeptCap.  Each lane first takes its entries of the four
// lists into registers (entry lane + 64 i of list w in slot [w][i], PL slots per list, key 0 in
// slots past a list's end), so that the bit-by-bit selections below are register compares and
// ballots, with no LDS traffic per bit; row_merge_lists picks the smallest PL that holds the
// longest list.
template <class E, int PL>
__device__ int row_merge_slots(const Samp& sp, int r, const Workspace& ws, RowLds& S) {
  constexpr int KB = Tr<E>::kKeyBits;
  const int lane = lane_id();
  int cnt[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) cnt[w] = S.cnt[w];
  uint32_t kr[4][PL];  // canonical keys of this lane's entries; 0 = no entry (valid keys are >= 1)
  uint32_t mk = 0, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int j = lane + 64 * i;
      kr[w][i] = j < cnt[w] ? S.key[w][j] : 0u;
      mk = kr[w][i] > mk ? kr[w][i] : mk;
      if (j < cnt[w]) lo = kr[w][i] < lo ? kr[w][i] : lo;
    }
  mk = wave_reduce(mk, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  lo = wave_reduce(lo, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
  const float m = Tr<E>::key_to_float(mk);
  auto count_ge = [&](uint32_t v) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int i = 0; i < PL; ++i) c += __popcll(__ballot(kr[w][i] >= v));
    return c;
  };
  // the k-th largest key, ties counted: the largest x with at least k entries >= x.  It lies
  // in [lo, mk] (at least k entries exist), so it shares their common high bits; the search
  // runs over the bits below.
  int hb = lo <= mk ? 31 - __builtin_clz((lo ^ mk) | 1u) : KB - 1;
  uint32_t x = lo <= mk ? lo & ~((2u << hb) - 1u) : 0u;
  if (hb == 31) x = 0u;
  for (int bit = hb; bit >= 0; --bit) {
    const uint32_t cand = x | (1u << bit);
    if (count_ge(cand) >= sp.top_k) x = cand;
  }
  if (x < 1u) x = 1u;  // key 0 marks no entry
  const float it = sp.inv_t;
  double part = 0.0;  // the top-k set's sum of exp((z - m) / T)
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < PL; ++i)
      if (kr[w][i] >= x) part += (double)fast_exp((Tr<E>::key_to_float(kr[w][i]) - m) * it);
  double Ssum = wave_reduce(part, [](double a, double b) { return a + b; });
  // the top-k set (every entry >= x) compacted into LDS in slot order
  const unsigned long long below = lanes_below();
  int nk = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const bool keep = kr[w][i] >= x;
      const unsigned long long mkp = __ballot(keep);
      const int pos = nk + __popcll(mkp & below);
      if (keep && pos < kKeptCap) {
        S.ckey[pos] = kr[w][i];
        S.cidx[pos] = S.idx[w][lane + 64 * i];
      }
      nk += __popcll(mkp);
    }
  if (nk > kKeptCap) return 1;
  wave_lds_sync();
  uint32_t tkey = x;
  if (sp.top_p < 1.0f) {
    if (nk <= 128)
      topp_compact<E, 2>(sp, S, nk, m, Ssum, tkey);
    else if (nk <= 320)
      topp_compact<E, 5>(sp, S, nk, m, Ssum, tkey);
    else
      topp_compact<E, kKeptCap / 64>(sp, S, nk, m, Ssum, tkey);
  }
  uint2* dst = ws.kept + (size_t)r * kKeptCap;
  int base = 0;
  for (int j0 = 0; j0 < nk; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t kj = j < nk ? S.ckey[j] : 0u;
    const bool keep = kj >= tkey;
    const unsigned long long mkp = __ballot(keep);
    if (keep)
      dst[base + __popcll(mkp & below)] =
          make_uint2(S.cidx[j], __float_as_uint(Tr<E>::key_to_float(kj)));
    base += __popcll(mkp);
  }
  if (lane == 0) {
    RowStat rs;
    rs.m = m;
    rs.thr = Tr<E>::key_to_float(tkey);
    rs.S = Ssum;
    rs.argmax = -1;
    rs.nkept = base;
    rs.kind = kRowCompact;
    rs.pad = 0;
    ws.rstat[r] = rs;
  }
  return 0;
}

template <class E>
__device__ int row_merge_lists(const Samp& sp, int r, const Workspace& ws, RowLds& S) {
  const int longest = max(max(S.cnt[0], S.cnt[1]), max(S.cnt[2], S.cnt[3]));
  if (longest <= 128) return row_merge_slots<E, 2>(sp, r, ws, S);
  if (longest <= 256) return row_merge_slots<E, 4>(sp, r, ws, S);
  if constexpr (Tr<E>::kKeyBits == 16)  // (with 32-bit keys this instantiation spills)
    if (longest <= 384) return row_merge_slots<E, 6>(sp, r, ws, S);
  return row_merge_slots<E, kWaveListCap / 64>(sp, r, ws, S);
}

// Whole-row fallback (all threads) when the candidates do not fit: the row maximum and exact
// selections by re-reading the row, 8-bit radix digits (2 KB of bins).  Writes a dense RowStat.
template <class E, bool VEC>
__device__ void row_merge_block(const E* __restrict__ row, const Dims& dm, const Samp& sp, int r,
                                const Workspace& ws, unsigned long long* s_bins,
                                RedScratch& red) {
  float mx = -INFINITY;
  row_foreach<E, VEC>(row, dm.V, [&](int, float z, uint32_t) { mx = fmaxf(mx, z); });
  const float m = block_max_f(mx, red);
  const float it = sp.inv_t;
  uint32_t key = radix_select<E, VEC, false, 8>(row, dm.V, m, it, 0u, (double)sp.top_k, s_bins);
  if (sp.top_p < 1.0f)
    key = radix_select<E, VEC, true, 8>(row, dm.V, m, it, key, (double)sp.top_p, s_bins);
  const float thr = Tr<E>::key_to_float(key);
  const double S = dense_sum<E, VEC>(row, dm.V, m, it, thr, red);
  if (threadIdx.x == 0) {
    RowStat rs;
    rs.m = m;
    rs.thr = thr;
    rs.S = S;
    rs.argmax = -1;
    rs.nkept = -1;
    rs.kind = kRowDense;
    rs.pad = 0;
    ws.rstat[r] = rs;
  }
}

// One workgroup per row, the row streamed in register tiles of 16-byte vectors.  A row need not
// start on a 16-byte boundary (e.g. an odd bf16 vocabulary): the vectors cover the aligned
// interior [h, h + nin) of the row, and the at most 2 (EPV - 1) elements before and after it
// (the fringe) are loaded one by one and appended to wave 0's list whatever their value.
// Tile 0 sets tau = the k-th largest of the 256 per-thread maxima (at most the tile's k-th
// largest, so at most the row's); every tile appends its elements >= tau to the wave's list,
// and a wave raises tau to its own list's k-th largest whenever the list grows long.  No
// barrier after tile 0.  At the end one wave selects the row's k-th largest among the
// candidates (the row's top-k set, ties included, is among them).
template <class E, bool GROUPS4>
__global__ __launch_bounds__(kThreads, 5) void k_topk_row(const E* __restrict__ tgt,
                                                       const E* __restrict__ drf, Dims dm,
                                                       Samp sp, Workspace ws, int targets_only) {
  constexpr int EPV = Tr<E>::kEpv;
  // targets_only: the grid covers the B (K+1) target rows (the draft rows' summaries are given)
  const int nr = targets_only ? dm.B * (dm.K + 1) : dm.rows;
  const int ri = xcd_contiguous((int)blockIdx.x, nr);
  const int r = targets_only ? target_row(dm, ri / (dm.K + 1), ri % (dm.K + 1)) : ri;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  __shared__ RowLds S;
  const E* row = row_ptr(dm, tgt, drf, r);
  const int V = dm.V;
  // elements before the first 16-byte boundary, the aligned interior, where the tail starts
  const int h = min(V, (int)(((16u - ((uint32_t)reinterpret_cast<uintptr_t>(row) & 15u)) & 15u) /
                             sizeof(E)));
  const int nin = (V - h) / EPV * EPV;
  const int tail = h + nin;
  const E* inner = row + h;
  const int ntiles = max(1, (nin + dm.chunk_elems - 1) / dm.chunk_elems);
  const int k = sp.top_k;
  const int raise_at = k + 128;  // a pass pushes at most 128, so lists stay within the cap
  WaveList L{wv, 0, 0, 0u};
  for (int c = 0; c < ntiles; ++c) {
    const int c0 = c * dm.chunk_elems;
    const int clen = min(dm.chunk_elems, nin - c0);
    uint32_t regs[kRegs];
    load_tile<E>(inner, c0, clen, regs);
    unsigned long long valid[kVecPerThread];
    tile_valid<E>(clen, valid);
    if (c == 0) {
      // Maxima of disjoint groups of the tile: the k-th largest of them is at most the tile's
      // k-th largest.  One group per thread (256 maxima), or with GROUPS4 (top-k above 64) four
      // per thread (registers [16 g, 16 g + 16), 1024 maxima in the still empty lists), whose
      // k-th largest lies much closer to the tile's and so admits far fewer candidates; that
      // variant is a kernel of its own, as its selection needs more registers.
      constexpr bool groups4 = GROUPS4;
      uint32_t* gm = &S.key[0][0];
      if constexpr (groups4) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t tm = 0;
#pragma unroll
          for (int j = 16 * g; j < 16 * g + 16; ++j)
            tm = Tr<E>::dword_max(tm, tile_key<E>(regs, j, valid));
          gm[g * kThreads + tid] = Tr<E>::dword_hmax(tm);
        }
      } else {
        uint32_t tm = 0;
#pragma unroll
        for (int j = 0; j < kRegs; ++j) tm = Tr<E>::dword_max(tm, tile_key<E>(regs, j, valid));
        S.tmax[tid] = Tr<E>::dword_hmax(tm);
      }
      // Opaque to the compiler, so that it recomputes the keys in filter_tile rather than
      // keeping all 64 of them live across the selection below.
#pragma unroll
      for (int j = 0; j < kRegs; ++j) asm volatile("" : "+v"(regs[j]));
      __syncthreads();
      if (wv == 0) {
        uint32_t x = 0;
        if constexpr (groups4) {
          uint32_t a[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) a[i] = gm[lane + 64 * i];
          for (int bit = Tr<E>::kKeyBits - 1; bit >= 0; --bit) {
            const uint32_t cand = x | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) cnt += __popcll(__ballot(a[i] >= cand));
            if (cnt >= k) x = cand;
          }
        } else {
          const uint32_t a0 = S.tmax[lane], a1 = S.tmax[lane + 64];
          const uint32_t a2 = S.tmax[lane + 128], a3 = S.tmax[lane + 192];
          for (int bit = Tr<E>::kKeyBits - 1; bit >= 0; --bit) {
            const uint32_t cand = x | (1u << bit);
            const int cnt = __popcll(__ballot(a0 >= cand)) + __popcll(__ballot(a1 >= cand)) +
                            __popcll(__ballot(a2 >= cand)) + __popcll(__ballot(a3 >= cand));
            if (cnt >= k) x = cand;
          }
        }
        if (lane == 0) {
          S.tau = filter_tau<E>(x);
#pragma unroll
          for (int w = 0; w < 4; ++w) S.wtau[w] = S.tau;
        }
      }
      __syncthreads();
      L.tau = S.tau;
      filter_tile<E, true>(regs, h + c0, valid, S, L, k, raise_at);
    } else if ((wl_shared_tau(S, L), L.tau > Tr<E>::kKeyPos0)) {
      filter_tile<E, false>(regs, h + c0, valid, S, L, k, raise_at);
    } else {
      filter_tile<E, true>(regs, h + c0, valid, S, L, k, raise_at);
    }
  }
  if (wv == 0 && nin < V) {  // the fringe, one element per lane
    if (L.count > raise_at) wl_raise<E>(S, L, k);
    const int f = lane < h ? lane : tail + (lane - h);
    uint32_t key = 0u;
    if (lane < V - nin) key = Tr<E>::key_of_bits(Tr<E>::bits_of(row[f]));
    wl_push(S, L, key != 0u, (uint32_t)f, Tr<E>::canon(key), false, 0u, 0u);
  }
  if (lane == 0) {
    S.cnt[wv] = L.count < kWaveListCap ? L.count : kWaveListCap;
    S.ovf[wv] = L.ovf | (L.count > kWaveListCap);
  }
  __syncthreads();
  if (wv == 0) {
    const int ovf = S.ovf[0] | S.ovf[1] | S.ovf[2] | S.ovf[3];
    const int fb = ovf ? 1 : row_merge_lists<E>(sp, r, ws, S);
    if (lane == 0) S.fallback = fb;
  }
  __syncthreads();
  if (S.fallback) {
    unsigned long long* bins = reinterpret_cast<unsigned long long*>(&S.key[0][0]);
    if (nin == V)  // the whole row is 16-byte aligned
      row_merge_block<E, true>(row, dm, sp, r, ws, bins, S.red);
    else
      row_merge_block<E, false>(row, dm, sp, r, ws, bins, S.red);
  }
}

// Row summaries of the draft rows taken from a spec_sample call on them (row b*K + k there):
// RowStat and, for compact rows, the kept list, into the verify workspace's draft rows.
__global__ __launch_bounds__(64) void k_take_draft_summaries(Dims dm, Workspace src,
                                                             Workspace ws) {
  const int pos = blockIdx.x;  // b * K + k
  const int b = pos / dm.K, k = pos - b * dm.K;
  const int dst = draft_row(dm, b, k);
  const RowStat rs = src.rstat[pos];
  if (threadIdx.x == 0) ws.rstat[dst] = rs;
  if (rs.kind == kRowCompact) {
    const uint2* from = src.kept + (size_t)pos * kKeptCap;
    uint2* to = ws.kept + (size_t)dst * kKeptCap;
    for (int e = threadIdx.x; e < rs.nkept; e += 64) to[e] = from[e];
  }
}

// Inverse-CDF pick over weights staged in LDS by one wave (s_idx / s_w, nk entries, total W):
// the smallest index whose cumulative weight in index order exceeds u * W; the largest index of
// positive weight if rounding leaves none.
// The same pick over at most 64 entries held one per lane (lane e: index ie, weight we; lanes
// >= nk hold none): each lane reads the others' entries in order and sums the weights of those
// at or below its own index; the smallest index whose sum exceeds u W is the token.
__device__ int pick_lanes(int nk, uint32_t ie, double we, double W, double u) {
  const int lane = lane_id();
  const double target = u * W;
  double pre = 0.0;
  for (int j = 0; j < nk; ++j) {
    const uint32_t ij = (uint32_t)__builtin_amdgcn_readlane((int)ie, j);
    const double wj = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(we), j),
                                       __builtin_amdgcn_readlane(__double2loint(we), j));
    if (ij <= ie) pre += wj;
  }
  uint32_t pick = 0xFFFFFFFFu;
  int lastpos = -1;
  if (lane < nk && we > 0.0) {
    if (pre > target) pick = ie;
    lastpos = (int)ie;
  }
  pick = wave_reduce(pick, [](uint32_t a, uint32_t c) { return a < c ? a : c; });
  lastpos = wave_reduce(lastpos, [](int a, int c) { return a > c ? a : c; });
  return pick != 0xFFFFFFFFu ? (int)pick : lastpos;
}

__device__ int pick_staged_wave(int nk, double W, double u, const uint32_t* s_idx,
                                const double* s_w) {
  wave_lds_sync();
  const double target = u * W;
  uint32_t pick = 0xFFFFFFFFu;
  int lastpos = -1;
  if (nk <= 64) {  // one entry per lane
    const int lane = lane_id();
    const int tok = pick_lanes(nk, lane < nk ? s_idx[lane] : 0xFFFFFFFFu,
                               lane < nk ? s_w[lane] : 0.0, W, u);
    wave_lds_sync();
    return tok;
  }
  // More entries than lanes: the smallest index i with C(i) > u W, C(i) = the weight of the
  // entries with index <= i, by bisection on i.  C is summed per lane in a fixed order and then
  // over the lanes in a fixed tree, both additions of non-negative terms, so it does not
  // decrease as i grows and the bisection finds the index a scan in index order would.
  for (int e = lane_id(); e < nk; e += 64)
    if (s_w[e] > 0.0 && (int)s_idx[e] > lastpos) lastpos = (int)s_idx[e];
  lastpos = wave_reduce(lastpos, [](int a, int c) { return a > c ? a : c; });
  auto C = [&](uint32_t i) {
    double t = 0.0;
    for (int e = lane_id(); e < nk; e += 64)
      if (s_idx[e] <= i) t += s_w[e];
    return wave_reduce(t, [](double a, double c) { return a + c; });
  };
  if (lastpos >= 0 && C((uint32_t)lastpos) > target) {  // else rounding: the last index
    uint32_t a = 0, c = (uint32_t)lastpos;
    while (a < c) {
      const uint32_t mid = a + (c - a) / 2;
      if (C(mid) > target)
        c = mid;
      else
        a = mid + 1;
    }
    pick = a;
  }
  wave_lds_sync();
  return pick != 0xFFFFFFFFu ? (int)pick : lastpos;
}

// Final draw over at most 64 kept tokens held one per lane (lane e < nk: index ie, target logit
// zt, draft logit zd): weights and order of additions as in final_draw_compact_wave.
__device__ int draw_small_wave(int nk, uint32_t ie, float zt, float zd, const RowStat& rt,
                               const RowStat& rd, bool resid, float it, double u) {
  const bool has = lane_id() < nk;
  const double q = has ? (double)fast_exp((zt - rt.m) * it) / rt.S : 0.0;
  double w = q;
  if (resid) {
    const double p = has ? (double)kept_exp(zd, rd, it) / rd.S : 0.0;
    w = q - p > 0.0 ? q - p : 0.0;
  }
  double W = wave_reduce(w, [](double a, double c) { return a + c; });
  if (!(W > 0.0)) {  // empty residual: draw from q
    w = q;
    W = wave_reduce(q, [](double a, double c) { return a + c; });
  }
  return pick_lanes(nk, has ? ie : 0xFFFFFFFFu, w, W, u);
}

// Final draw over a compact row, one wave.  Weights (q - p)_+ (or q for the bonus row, or q
// when the residual is empty); the token is the smallest index whose cumulative weight in
// index order exceeds u * W.  Entries are staged in LDS (s_idx / s_w).
template <class E>
__device__ int final_draw_compact_wave(const E* __restrict__ tgt, const E* __restrict__ drf,
                                       const Dims& dm, const Samp& sp, const Workspace& ws, int b,
                                       int n, const RowStat& rt, const RowStat& rd, double u,
                                       uint32_t* s_idx, double* s_w) {
  const int lane = lane_id();
  const int nk = rt.nkept;
  const uint2* kept = ws.kept + (size_t)target_row(dm, b, n) * kKeptCap;
  const bool resid = n < dm.K;
  const E* drow = resid ? row_ptr(dm, tgt, drf, draft_row(dm, b, n)) : nullptr;
  const float it = sp.inv_t;
  if (nk <= 64) {
    uint32_t ie = 0xFFFFFFFFu;
    float zt = 0.0f, zd = 0.0f;
    if (lane < nk) {
      const uint2 v = kept[lane];
      ie = v.x;
      zt = __uint_as_float(v.y);
      if (resid) zd = Tr<E>::to_float(Tr<E>::bits_of(drow[v.x]));
    }
    return draw_small_wave(nk, ie, zt, zd, rt, rd, resid, it, u);
  }
  // entries lane + 64 i, four per lane at a time: the four kept entries, then the four draft
  // logits at their indices, are loaded together (two round trips per 256 entries, not two per
  // entry); the weights are added in entry order
  double Wp = 0.0;
  for (int e0 = 0; e0 < nk; e0 += 256) {
    uint2 v[4];
    float zd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + lane + 64 * i;
      v[i] = e < nk ? kept[e] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + lane + 64 * i;
      zd[i] = (resid && e < nk) ? Tr<E>::to_float(Tr<E>::bits_of(drow[v[i].x])) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + lane + 64 * i;
      if (e < nk) {
        const double q = (double)fast_exp((__uint_as_float(v[i].y) - rt.m) * it) / rt.S;
        double w = q;
        if (resid) {
          const double p = (double)kept_exp(zd[i], rd, it) / rd.S;
          w = q - p > 0.0 ? q - p : 0.0;
        }
        s_idx[e] = v[i].x;
        s_w[e] = w;
        Wp += w;
      }
    }
  }
  double W = wave_reduce(Wp, [](double a, double c) { return a + c; });
  if (!(W > 0.0)) {  // empty residual: draw from q
    double Qp = 0.0;
    for (int e = lane; e < nk; e += 64) {
      const double q = (double)fast_exp((__uint_as_float(kept[e].y) - rt.m) * it) / rt.S;
      s_w[e] = q;
      Qp += q;
    }
    W = wave_reduce(Qp, [](double a, double c) { return a + c; });
  }
  return pick_staged_wave(nk, W, u, s_idx, s_w);
}

// ------------------------------------------------------------------------------------------
// Mentored decoding (community blog on an optimal lossy variant of speculative decoding,
// sections on mentored decoding and on solving the optimisation problem).  Per draft position,
// over the target's kept tokens (q_i > 0): r_i = min(1, q_i / (alpha p_i)) and replacement
// weights w_i = max(0, q_i / beta - p_i), beta making the emitted law pi = p r + w sum to 1,
// alpha the smallest value on the grid of 50 halvings of [0, 1] with KL(q || pi) <= D.
//
// With the tokens sorted by ratio q_i / p_i (decreasing), and ia = #{ratio >= alpha}, the
// active set of the replacement is a prefix of m tokens (all with ratio > beta >= alpha), and
//   sum_i p_i r_i = P[ia] + (Q[n] - Q[ia]) / alpha,   beta = Q[m] / (R + P[m]),
//   KL = Q[m] ln beta + (L[ia] - L[m]) + (Q[n] - Q[ia]) ln alpha
// with prefix sums Q, P, L of q, p and q ln(q / p) in that order: pi_i = q_i / beta on the
// prefix, p_i up to ia, q_i / alpha after it.  These are the precomputed sums the blog lists.
// m is the first prefix length whose beta reaches the next ratio; that condition, once met,
// holds for every longer prefix (beta of a longer prefix lies between the shorter one's beta
// and the added ratio), so both ia and m are binary searches.
//
// The grid point is found by multisection: KL decreases in alpha, so the smallest grid point
// with KL <= D is the one bisection reaches; each round evaluates 64 evenly spaced grid points
// of the current interval in parallel, one per lane, and keeps the sub-interval in front of
// the first point that satisfies the bound (9 rounds instead of 50 dependent steps).
// ------------------------------------------------------------------------------------------
template <int CAP>
struct MentorLds {
  double r[CAP];                // ratios, sorted in decreasing order (-1: no entry)
  double q[CAP], p[CAP];        // by kept-list position
  double lq[CAP];               // q ln(q / p) by kept-list position (0 where p = 0)
  double qc[CAP + 1], pc[CAP + 1], lc[CAP + 1];  // prefix sums, sorted order
  uint16_t pos[CAP];            // kept-list position of each sorted entry
};

constexpr int kMentorSmallCap = 256;  // kept tokens the first mentored pass holds in LDS

// q_i or p_i of a kept logit in fp64, evaluated as exp(z/T - m/T) / S (the order the
// probabilities are defined in: scale by the temperature, subtract the maximum, normalise).
__device__ __forceinline__ double prob64(float z, float m, double T, double S) {
  return exp((double)z / T - (double)m / T) / S;
}

// Does (ra, pa) precede (rb, pb) in decreasing ratio order (ties: lower kept position first)?
__device__ __forceinline__ bool ratio_before(double ra, uint32_t pa, double rb, uint32_t pb) {
  return ra > rb || (ra == rb && pa < pb);
}

// m = the first prefix length with Q[m] / (R + P[m]) >= the next ratio, searched in [lo, hi]
// (hi qualifies: the full support always does); R > 0.
template <int CAP>
__device__ int mentor_m_search(const MentorLds<CAP>& L, int lo, int hi, double R) {
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (L.qc[mid] / (R + L.pc[mid]) >= L.r[mid])
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// KL(q || pi_alpha) of one lane's alpha, from the sorted ratios and prefix sums; beta out.
// ia and m (-1 when R <= 0, where no prefix is active) are returned for reuse: ia falls and m
// rises with alpha, so when they agree at the two ends of an interval they hold inside it,
// and `hint` (ia >= 0) skips the searches; otherwise the searches run between the values at
// the ends, ia in [ia_min, ia_max] and m in [m_min, m_max].
template <int CAP>
__device__ double mentor_kl_at(const MentorLds<CAP>& L, int nsup, int ninf, double alpha,
                               int hint_ia, int hint_m, int ia_min, int ia_max, int m_min,
                               int m_max, int& ia_out, int& m_out, double& beta) {
  int ia = hint_ia;
  if (ia < 0) {  // ia = #{ratio >= alpha}
    int lo = ia_min, hi = ia_max;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (L.r[mid] >= alpha)
        lo = mid + 1;
      else
        hi = mid;
    }
    ia = lo;
  }
  ia_out = ia;
  const double qn = L.qc[nsup];
  const double qlo = qn - L.qc[ia];
  const double R = 1.0 - (L.pc[ia] + qlo / alpha);
  const double lna = log(alpha);
  if (!(R > 0.0)) {  // no replacement mass: pi = p r
    m_out = -1;
    beta = INFINITY;
    return ninf > 0 ? INFINITY : L.lc[ia] + qlo * lna;
  }
  int m = hint_ia >= 0 ? hint_m : -1;
  if (m < 0) m = mentor_m_search(L, m_min, m_max, R);
  m_out = m;
  beta = L.qc[m] / (R + L.pc[m]);
  const double lnb = log(beta);
  if (m <= ia) return L.qc[m] * lnb + (L.lc[ia] - L.lc[m]) + qlo * lna;
  // rounding put tokens with ratio < alpha into the active prefix: their pi_i is
  // q_i / alpha + q_i / beta - p_i
  double odd = 0.0;
  for (int j = ia; j < m; ++j) {
    const int e = L.pos[j];
    const double q = L.q[e];
    odd += q * log(q / (q / alpha + (q / beta - L.p[e])));
  }
  return L.qc[ia] * lnb + odd + (qn - L.qc[m]) * lna;
}

// Solve of draft position `pos` (= b * K + k) by one wave.  CAP = kMentorSmallCap: positions
// whose target row keeps more tokens are marked kMentorDeferred and solved with CAP = kKeptCap
// by the sequence's block of k_seq_compact.
template <class E, int CAP>
__device__ void mentor_solve_wave(const E* __restrict__ tgt, const E* __restrict__ drf,
                                  const Dims& dm, const Samp& sp, const Workspace& ws,
                                  const int32_t* __restrict__ drafts,
                                  const float* __restrict__ uni, int need_all, int pos,
                                  MentorLds<CAP>& L) {
  const int lane = lane_id();
  const int K = dm.K;
  const int b = pos / K;
  const int k = pos - b * K;
  MentorSol* out = ws.ment + pos;
  const int ti = target_row(dm, b, k), di = draft_row(dm, b, k);
  const RowStat rt = ws.rstat[ti], rd = ws.rstat[di];
  MentorSol sol;
  sol.a = 0.0;
  sol.qx = 0.0;
  sol.px = 0.0;
  sol.alpha = 1.0;
  sol.beta = INFINITY;
  sol.st = 0.0;
  sol.sd = 0.0;
  sol.mode = kMentorLossless;
  sol.pad = 0;
  if (rt.kind != kRowCompact || rd.kind != kRowCompact) {
    if (lane == 0) *out = sol;
    return;
  }
  const int n = rt.nkept;
  if (n > CAP) {  // only in the small pass: the kKeptCap pass holds any kept list
    sol.mode = kMentorDeferred;
    if (lane == 0) *out = sol;
    return;
  }
  const double T = (double)sp.temperature;
  const double D = sp.mentor_d;
  const uint2* kt = ws.kept + (size_t)ti * kKeptCap;
  const uint2* kd = ws.kept + (size_t)di * kKeptCap;

  // the draft token's logits, loaded first so that their latency overlaps the sums below
  const E* trow = row_ptr(dm, tgt, drf, ti);
  const E* drow = row_ptr(dm, tgt, drf, di);
  const int x = drafts[(size_t)b * K + k];
  const double u = (double)uni[(size_t)b * (K + 1) + k];
  const bool x_in = x >= 0 && x < dm.V;
  const float zt_x = x_in ? load_logit(trow, x) : -INFINITY;
  const float zd_x = x_in ? load_logit(drow, x) : -INFINITY;

  // fp64 normalisers over the kept sets; the target's terms are kept for q below
  double st = 0.0, sd = 0.0;
  for (int e = lane; e < n; e += 64) {
    const double ex = exp((double)__uint_as_float(kt[e].y) / T - (double)rt.m / T);
    L.q[e] = ex;
    st += ex;
  }
  for (int e = lane; e < rd.nkept; e += 64)
    sd += exp((double)__uint_as_float(kd[e].y) / T - (double)rd.m / T);
  st = wave_reduce(st, [](double a, double c) { return a + c; });
  sd = wave_reduce(sd, [](double a, double c) { return a + c; });
  sol.st = st;
  sol.sd = sd;

  // q and p of the draft token and the lossless acceptance min(1, q/p), a lower bound of r
  double qx = 0.0, px = 0.0;
  if (x_in) {
    if (zt_x >= rt.thr) qx = prob64(zt_x, rt.m, T, st);
    if (zd_x >= rd.thr) px = prob64(zd_x, rd.m, T, sd);
  }
  sol.qx = qx;
  sol.px = px;
  const double a0 = px > 0.0 ? fmin(1.0, qx / px) : (qx > 0.0 ? 1.0 : 0.0);
  if (!need_all && u < a0) {
    sol.a = a0;
    sol.mode = kMentorShortcut;
    if (lane == 0) *out = sol;
    return;
  }

  // entries of the target support: q, p, ratio; KL(q || p)
  double klp = 0.0;
  int nsup = 0;
  double my_r = -1.0;  // ratio of this lane's entry (the only one when n <= 64)
  for (int e0 = 0; e0 < n; e0 += 64) {
    const int e = e0 + lane;
    bool sup = false;
    if (e < n) {
      const uint2 v = kt[e];
      const double q = L.q[e] / st;  // = prob64 of the target logit (same exponential)
      const float zd = load_logit(drow, (int)v.x);
      const double p = zd >= rd.thr ? prob64(zd, rd.m, T, sd) : 0.0;
      sup = q > 0.0;
      my_r = !sup ? -1.0 : (p > 0.0 ? q / p : INFINITY);
      const double lq = sup && p > 0.0 ? q * log(my_r) : 0.0;
      L.q[e] = q;
      L.p[e] = p;
      L.r[e] = my_r;
      L.lq[e] = lq;
      L.pos[e] = (uint16_t)e;
      if (sup) klp += p > 0.0 ? lq : INFINITY;
    }
    nsup += __popcll(__ballot(sup));
  }
  klp = wave_reduce(klp, [](double a, double c) { return a + c; });
  if (klp <= D) {
    sol.a = (qx > 0.0 || px > 0.0) ? 1.0 : 0.0;
    sol.alpha = 0.0;
    sol.mode = kMentorTrivial;
    if (lane == 0) *out = sol;
    return;
  }

  // sort (ratio, position) into decreasing ratio order (ties: lower position first)
  if (n <= 64) {
    // one entry per lane: its rank from the other entries' ratios (broadcast LDS reads)
    wave_lds_sync();
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += ratio_before(L.r[j], (uint32_t)j, my_r, (uint32_t)lane);
    wave_lds_sync();
    if (lane < n) {
      L.r[rank] = my_r;
      L.pos[rank] = (uint16_t)lane;
    }
  } else {  // bitonic sort over a power-of-two span
    int N = 2;
    while (N < n) N <<= 1;
    for (int e = n + lane; e < N; e += 64) {
      L.r[e] = -1.0;
      L.pos[e] = 0xFFFFu;
    }
    for (int size = 2; size <= N; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        wave_lds_sync();
        for (int t = lane; t < (N >> 1); t += 64) {
          const int i = ((t & ~(stride - 1)) << 1) | (t & (stride - 1));
          const int l = i + stride;
          const double ri = L.r[i], rl = L.r[l];
          const uint32_t pi = L.pos[i], pl = L.pos[l];
          const bool swap = (i & size) == 0 ? ratio_before(rl, pl, ri, pi)
                                            : ratio_before(ri, pi, rl, pl);
          if (swap) {
            L.r[i] = rl;
            L.r[l] = ri;
            L.pos[i] = (uint16_t)pl;
            L.pos[l] = (uint16_t)pi;
          }
        }
      }
  }
  wave_lds_sync();

  // prefix sums over the nsup support entries in sorted order: each lane a contiguous segment
  const int seg = (nsup + 63) >> 6;
  const int j0 = lane * seg, j1 = min(nsup, j0 + seg);
  double aq = 0.0, ap = 0.0, al = 0.0;
  for (int j = j0; j < j1; ++j) {
    const int e = L.pos[j];
    aq += L.q[e];
    ap += L.p[e];
    al += L.lq[e];
  }
  double iq = aq, ip = ap, il = al;  // inclusive scans over lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double tq = __shfl_up(iq, o), tp = __shfl_up(ip, o), tl = __shfl_up(il, o);
    if (lane >= o) {
      iq += tq;
      ip += tp;
      il += tl;
    }
  }
  double cq = __shfl_up(iq, 1), cp = __shfl_up(ip, 1), cl = __shfl_up(il, 1);
  if (lane == 0) {
    cq = 0.0;
    cp = 0.0;
    cl = 0.0;
    L.qc[0] = 0.0;
    L.pc[0] = 0.0;
    L.lc[0] = 0.0;
  }
  for (int j = j0; j < j1; ++j) {
    const int e = L.pos[j];
    cq += L.q[e];
    cp += L.p[e];
    cl += L.lq[e];
    L.qc[j + 1] = cq;
    L.pc[j + 1] = cp;
    L.lc[j + 1] = cl;
  }
  wave_lds_sync();
  int ninf = 0;
  for (int c0 = 0; c0 < nsup; c0 += 64)
    ninf += __popcll(__ballot(c0 + lane < nsup && L.r[c0 + lane] == INFINITY));

  // Search on the grid of 2^-kMentorBisectionSteps, in grid units: (LO, HI] holds the answer
  // and HI satisfies the bound (HI = 1 is taken to, as bisection never tests it).  Each round
  // evaluates up to 64 grid points inside (LO, HI), one per lane, and keeps HI = the smallest
  // point that satisfies the bound and LO = the largest point below it that does not (KL
  // decreases in alpha, so this is the interval bisection would narrow to).  The first round,
  // and any round without the KL values at both ends, spreads all 64 points evenly; later
  // rounds spread 16 points evenly (at least a 16-fold cut) and put 48 at a spacing of 1/2048
  // of the interval around the point where the straight line through the two ends' KL values
  // meets D, which is where the answer lies once the interval is short.
  const double grid = ldexp(1.0, -kMentorBisectionSteps);
  double LO = 0.0, HI = ldexp(1.0, kMentorBisectionSteps);  // integers, exact in fp64
  double kl_lo = NAN, kl_hi = NAN;
  // ia and m at the two ends (-1: not known).  Near alpha = 0 every ratio is >= alpha, no q
  // mass is scaled (R = 1 - P[nsup]), so ia and m take their limits there.
  int ia_lo = nsup, m_lo = -1, ia_hi = -1, m_hi = -1;
  {
    const double R0 = 1.0 - L.pc[nsup];
    if (R0 > 0.0) m_lo = mentor_m_search(L, 1, nsup, R0);
  }
  double beta_hi = -1.0;  // beta at HI once a lane has evaluated it
  while (HI - LO > 1.0) {
    const double W = HI - LO;
    // both ends evaluated, KL finite at LO (KL at HI is <= D)
    const bool interp = kl_lo == kl_lo && kl_hi == kl_hi && kl_lo < INFINITY;
    double idx;
    if (!interp || lane < 16) {
      idx = LO + fmax(floor(W / (interp ? 16.0 : 64.0)), 1.0) * (double)(lane + 1);
    } else {
      const double c = LO + floor((kl_lo - D) / (kl_lo - kl_hi) * W);
      idx = c + fmax(floor(W * (1.0 / 2048.0)), 1.0) * (double)(lane - 40);
    }
    const bool inside = idx > LO && idx < HI;
    const bool same = ia_lo >= 0 && ia_lo == ia_hi && m_lo == m_hi;
    int ia = -1, m = -1;
    double bt = -1.0, kl = NAN;
    // ia between its values at HI and LO; m between those at LO and HI where known
    int ia_min = ia_hi >= 0 ? ia_hi : 0, ia_max = ia_lo >= 0 ? ia_lo : nsup;
    int m_min = m_lo >= 1 ? m_lo : 1, m_max = m_hi >= 1 ? m_hi : nsup;
    if (ia_min > ia_max) ia_min = 0, ia_max = nsup;  // (rounding at the ends: search it all)
    if (m_min > m_max) m_min = 1, m_max = nsup;
    if (inside)
      kl = mentor_kl_at(L, nsup, ninf, idx * grid, same ? ia_lo : -1, m_lo, ia_min, ia_max,
                        m_min, m_max, ia, m, bt);
    const bool ok = inside && kl <= D;
    // The points rise with the lane inside each group (lanes 0-63, or 0-15 and 16-63), so the
    // new ends come from ballots: HI from each group's first satisfying lane, LO from each
    // group's last failing lane before that (and below the new HI).
    const unsigned long long okm = __ballot(ok), failm = __ballot(inside && !ok);
    const unsigned long long groups[2] = {interp ? 0xFFFFull : ~0ull,
                                          interp ? ~0xFFFFull : 0ull};
    double nhi = HI;
    int fh = -1;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const unsigned long long gm = okm & groups[g];
      if (gm) {
        const int f = __ffsll((long long)gm) - 1;
        const double v = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(idx), f),
                                          __builtin_amdgcn_readlane(__double2loint(idx), f));
        if (v < nhi) {
          nhi = v;
          fh = f;
        }
      }
    }
    double nlo = LO;
    int fl = -1;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const unsigned long long okg = okm & groups[g];
      unsigned long long gm = failm & groups[g];
      if (okg) gm &= (1ull << (__ffsll((long long)okg) - 1)) - 1ull;  // lanes before the first ok
      if (gm) {
        const int l = 63 - __clzll((long long)gm);
        const double v = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(idx), l),
                                          __builtin_amdgcn_readlane(__double2loint(idx), l));
        if (v > nlo && v < nhi) {
          nlo = v;
          fl = l;
        }
      }
    }
    if (fh >= 0) {  // the lane holding the new HI
      ia_hi = __builtin_amdgcn_readlane(ia, fh);
      m_hi = __builtin_amdgcn_readlane(m, fh);
      beta_hi = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(bt), fh),
                                 __builtin_amdgcn_readlane(__double2loint(bt), fh));
      kl_hi = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(kl), fh),
                               __builtin_amdgcn_readlane(__double2loint(kl), fh));
    }
    if (fl >= 0) {  // the lane holding the new LO
      ia_lo = __builtin_amdgcn_readlane(ia, fl);
      m_lo = __builtin_amdgcn_readlane(m, fl);
      kl_lo = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(kl), fl),
                               __builtin_amdgcn_readlane(__double2loint(kl), fl));
    }
    LO = nlo;
    HI = nhi;
  }
  const double hi = HI * grid;
  double beta = beta_hi;
  if (beta < 0.0) {  // hi = 1, never evaluated
    int ia, m;
    (void)mentor_kl_at(L, nsup, ninf, hi, -1, -1, 0, nsup, 1, nsup, ia, m, beta);
  }
  sol.alpha = hi;
  sol.beta = beta;
  sol.a = px > 0.0 ? fmin(1.0, qx / (hi * px)) : (qx > 0.0 ? 1.0 : 0.0);
  sol.mode = kMentorSolved;
  if (lane == 0) *out = sol;
}

// First pass: one 64-thread block per draft position, kept lists up to kMentorSmallCap.
template <class E>
__global__ __launch_bounds__(64) void k_mentor(const E* __restrict__ tgt,
                                               const E* __restrict__ drf, Dims dm, Samp sp,
                                               Workspace ws, const int32_t* __restrict__ drafts,
                                               const float* __restrict__ uni, int need_all) {
  __shared__ MentorLds<kMentorSmallCap> L;
  mentor_solve_wave<E, kMentorSmallCap>(tgt, drf, dm, sp, ws, drafts, uni, need_all,
                                        (int)blockIdx.x, L);
}

// Final draw of a mentored position n < K, one wave: weights max(0, q_i / beta - p_i) over the
// target's kept tokens (q if they have no mass), fp64 with the solve's normalisers.
template <class E>
__device__ int mentor_draw_wave(const E* __restrict__ tgt, const E* __restrict__ drf,
                                const Dims& dm, const Samp& sp, const Workspace& ws, int b, int n,
                                const MentorSol& ms, double u, uint32_t* s_idx, double* s_w) {
  const int lane = lane_id();
  const RowStat rt = ws.rstat[target_row(dm, b, n)];
  const RowStat rd = ws.rstat[draft_row(dm, b, n)];
  const int nk = rt.nkept;
  const uint2* kept = ws.kept + (size_t)target_row(dm, b, n) * kKeptCap;
  const E* drow = row_ptr(dm, tgt, drf, draft_row(dm, b, n));
  const double T = (double)sp.temperature;
  const bool solved = ms.mode == kMentorSolved;
  double Wp = 0.0;
  for (int e = lane; e < nk; e += 64) {
    const uint2 v = kept[e];
    double w = 0.0;
    if (solved) {
      const double q = prob64(__uint_as_float(v.y), rt.m, T, ms.st);
      const float zd = load_logit(drow, (int)v.x);
      const double p = zd >= rd.thr ? prob64(zd, rd.m, T, ms.sd) : 0.0;
      w = q / ms.beta - p;
      w = w > 0.0 ? w : 0.0;
    }
    s_idx[e] = v.x;
    s_w[e] = w;
    Wp += w;
  }
  double W = wave_reduce(Wp, [](double a, double c) { return a + c; });
  if (!(W > 0.0)) {  // no replacement mass: draw from q
    double Qp = 0.0;
    for (int e = lane; e < nk; e += 64) {
      const double q = prob64(__uint_as_float(kept[e].y), rt.m, T, ms.st);
      s_w[e] = q;
      Qp += q;
    }
    W = wave_reduce(Qp, [](double a, double c) { return a + c; });
  }
  return pick_staged_wave(nk, W, u, s_idx, s_w);
}

// Final draw over a full row pair (all threads): totals, then a scan in index order.
template <class E, bool VEC>
__device__ int final_draw_dense_block(const E* __restrict__ trow, const E* __restrict__ drow,
                                      const RowStat& rt, const RowStat& rd, bool resid, float it,
                                      int V, double u, RedScratch& red, double* s_scan) {
  constexpr int EPV = Tr<E>::kEpv;
  const int tid = threadIdx.x;
  const int nvec = (V + EPV - 1) / EPV;
  double W = 0.0, Q = 0.0;
  for (int v = tid; v < nvec; v += kThreads) {
    float zt[EPV], zd[EPV];
    load_vec_f<E, VEC>(trow, V, v * EPV, zt);
    if (resid) load_vec_f<E, VEC>(drow, V, v * EPV, zd);
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      W += final_weight(zt[e], resid ? zd[e] : 0.f, rt, rd, resid, false, it);
      Q += final_weight(zt[e], 0.f, rt, rd, false, true, it);
    }
  }
  W = block_sum_d(W, red);
  Q = block_sum_d(Q, red);
  const bool use_q = !(W > 0.0) || !resid;
  const double target = u * (use_q ? Q : W);
  double carry = 0.0;
  int pick = INT_MAX, lastpos = -1;
  for (int v0 = 0; v0 < nvec; v0 += kThreads) {
    const int v = v0 + tid;
    double w[EPV];
    double local = 0.0;
    float zt[EPV], zd[EPV];
    if (v < nvec) {
      load_vec_f<E, VEC>(trow, V, v * EPV, zt);
      if (resid) load_vec_f<E, VEC>(drow, V, v * EPV, zd);
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      w[e] = (v < nvec) ? final_weight(zt[e], resid ? zd[e] : 0.f, rt, rd, resid, use_q, it) : 0.0;
      local += w[e];
    }
    s_scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const double add = tid >= off ? s_scan[tid - off] : 0.0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    double cum = carry + (s_scan[tid] - local);
    int mine = INT_MAX, mylast = -1;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      if (w[e] > 0.0) mylast = v * EPV + e;
      cum += w[e];
      if (mine == INT_MAX && cum > target && w[e] > 0.0) mine = v * EPV + e;
    }
    const double round_total = s_scan[kThreads - 1];
    const int got = block_min_i(mine, red);
    const int lp = block_max_i(mylast, red);
    if (lp > lastpos) lastpos = lp;
    if (got != INT_MAX) {
      pick = got;
      break;
    }
    carry += round_total;
  }
  return pick != INT_MAX ? pick : lastpos;
}

// LDS of k_seq_compact: the final draw's staging, or (mentored decoding) the solve of the
// positions whose kept lists were too long for k_mentor.
template <bool MENTOR>
struct SeqCompactLds {
  union {
    struct {
      double w[kKeptCap];
      uint32_t idx[kKeptCap];
    } draw;
    MentorLds<MENTOR ? kKeptCap : 1> ment;
  };
};


template <class E, bool VEC, bool MENTOR>
__global__ __launch_bounds__(kThreads) void k_seq_compact(const E* __restrict__ tgt,
                                                          const E* __restrict__ drf, Dims dm,
                                                          Samp sp, Workspace ws, Outs o) {
  const int b = blockIdx.x;
  const int K = dm.K;
  __shared__ SeqCompactLds<MENTOR> S;
  double* s_w = S.draw.w;
  uint32_t* s_idx = S.draw.idx;
  __shared__ int s_n, s_kind;
  __shared__ RedScratch red;
  const double u = (double)o.uni[(size_t)b * (K + 1) + K];
  if constexpr (MENTOR) {
    if (wave_id() == 0) {  // deferred mentored solves of this sequence, one at a time
      for (int k0 = 0; k0 < K; k0 += 64) {
        const int k = k0 + lane_id();
        unsigned long long def =
            __ballot(k < K && ws.ment[(size_t)b * K + k].mode == kMentorDeferred);
        while (def) {
          const int j = __ffsll((long long)def) - 1;
          def &= def - 1;
          mentor_solve_wave<E, kKeptCap>(tgt, drf, dm, sp, ws, o.drafts, o.uni,
                                         o.a != nullptr ? 1 : 0, b * K + k0 + j, S.ment);
          wave_lds_sync();  // the solution's store and the LDS reuse below
        }
      }
    }
  }
  if (wave_id() == 0) {
    LaneStats ls;
    const int n = seq_accept_wave<E>(tgt, drf, dm, sp, ws, o, b, ls);
    RowStat rt, rd;
    final_row_stats(dm, ws, b, n, ls, rt, rd);
    if (lane_id() == 0) {
      s_n = n;
      s_kind = rt.kind;
    }
    const MentorSol* ms = (sp.mentor && n < K) ? ws.ment + (size_t)b * K + n : nullptr;
    if (ms && ms->mode != kMentorLossless) {  // both rows compact: a wave draw
      const MentorSol sol = *ms;
      const int tok = mentor_draw_wave<E>(tgt, drf, dm, sp, ws, b, n, sol, u, s_idx, s_w);
      if (lane_id() == 0) o.tokens[(size_t)b * (K + 1) + n] = tok;
    } else if (rt.kind == kRowCompact) {
      const int tok =
          final_draw_compact_wave<E>(tgt, drf, dm, sp, ws, b, n, rt, rd, u, s_idx, s_w);
      if (lane_id() == 0) o.tokens[(size_t)b * (K + 1) + n] = tok;
    }
  }
  __syncthreads();
  if (s_kind != kRowCompact) {  // a row whose candidates overflowed: draw over the full rows
    const int n = s_n;
    const RowStat rt = ws.rstat[target_row(dm, b, n)];
    const bool resid = n < K;
    const RowStat rd = resid ? ws.rstat[draft_row(dm, b, n)] : rt;
    const E* trow = row_ptr(dm, tgt, drf, target_row(dm, b, n));
    const E* drow = resid ? row_ptr(dm, tgt, drf, draft_row(dm, b, n)) : trow;
    const int tok = final_draw_dense_block<E, VEC>(trow, drow, rt, rd, resid, sp.inv_t, dm.V, u,
                                                   red, s_w);
    if (threadIdx.x == 0) o.tokens[(size_t)b * (K + 1) + n] = tok;
  }
}

// ------------------------------------------------------------------------------------------
// Tree walk: one workgroup per sequence (REST article, section on retrieval-based speculative
// decoding: a node is accepted exactly when its parent is and its token is the argmax of the
// parent's target row).  Node argmaxes come from the chunk parts (first chunk wins ties, so the
// lowest index).  Acceptance is a conjunction along the path to the root, found for every node
// at once by pointer jumping: each node holds (ancestor a, distance d to it, ok = every edge
// from the node up to a matches); a round replaces it by (a of a, d + d of a, ok and ok of a),
// so after ceil(log2 N) rounds every ancestor is a terminal: the root (a self-loop with d = 0,
// ok = 1) or a node with an invalid parent (a self-loop with ok = 0).  A node is then accepted
// iff ok and d <= max_depth, d being its depth; the deepest accepted node, lowest index on
// ties, comes from one max-reduction, and its path is read back through the parents.
// ------------------------------------------------------------------------------------------
constexpr int kTreeMaxNodes = 2048;
constexpr int kTreeThreads = 256;
// (ancestor: bits 0-10, distance: bits 11-21, ok: bit 22) of a node
constexpr uint32_t kJumpA = 2047u, kJumpOk = 1u << 22;

// The same walk for trees of at most 64 nodes: one wave per sequence, node i in lane i; the
// pointer jumping runs on shuffles (no LDS, no barriers) and the path is read back by readlane.
__global__ __launch_bounds__(64) void k_tree_walk64(Dims dm, Workspace ws,
                                                    const int32_t* __restrict__ parent,
                                                    const int32_t* __restrict__ tokens,
                                                    int max_depth,
                                                    int32_t* __restrict__ out_tokens,
                                                    int32_t* __restrict__ out_n,
                                                    int32_t* __restrict__ out_last) {
  const int b = blockIdx.x;
  const int i = lane_id();
  const int N = dm.K;  // nodes per tree (stored in K for the tree launch), at most 64
  int g = 0, par = -1, tok = 0;
  if (i < N) {
    const ChunkPart* p = ws.parts + ((size_t)b * N + i) * dm.nchunks;
    float best = p[0].vmax;
    int am = p[0].argmax;
    for (int c = 1; c < dm.nchunks; ++c) {
      const float v = p[c].vmax;
      if (v > best) {
        best = v;
        am = p[c].argmax;
      }
    }
    g = am;
    par = parent[(size_t)b * N + i];
    tok = tokens[(size_t)b * N + i];
  }
  const bool valid = i > 0 && i < N && par >= 0 && par < i;
  const int gp = __shfl(g, valid ? par : 0);  // the parent's argmax
  // the root and the lanes past N are terminals (those lanes never accepted); an invalid parent
  // makes a terminal that is not ok
  uint32_t w = i == 0 ? kJumpOk
                      : valid ? (uint32_t)par | (1u << 11) | (tok == gp ? kJumpOk : 0u)
                              : (uint32_t)i;
  for (int span = 1; span < N; span <<= 1) {  // ceil(log2 N) rounds
    const uint32_t wa = (uint32_t)__shfl((int)w, (int)(w & kJumpA));
    const uint32_t d = ((w >> 11) & kJumpA) + ((wa >> 11) & kJumpA);
    w = (wa & kJumpA) | (d << 11) | (w & wa & kJumpOk);
  }
  // deepest accepted node, lowest index on ties (the root is always accepted)
  int key = 0;
  if (i < N) {
    const int d = (int)((w >> 11) & kJumpA);
    if ((w & kJumpOk) && d <= max_depth) key = (d << 11) | (2047 - i);
  }
  key = wave_reduce(key, [](int x, int y) { return x > y ? x : y; });
  const int best = 2047 - (key & 2047);
  const int depth = key >> 11;
  int32_t* o = out_tokens + (size_t)b * (max_depth + 1);
  for (int j = depth + 1 + i; j <= max_depth; j += 64) o[j] = -1;
  int cur = best;
  for (int j = depth - 1; j >= 0; --j) {  // the path, from best up to the root's child
    const int t = __builtin_amdgcn_readlane(tok, cur);
    if (i == 0) o[j] = t;
    cur = __builtin_amdgcn_readlane(par, cur);
  }
  if (i == 0) {
    o[depth] = __builtin_amdgcn_readlane(g, best);
    out_n[b] = depth;
    if (out_last) out_last[b] = best;
  }
}

__global__ __launch_bounds__(kTreeThreads) void k_tree_walk(Dims dm, Workspace ws,
                                                            const int32_t* __restrict__ parent,
                                                            const int32_t* __restrict__ tokens,
                                                            int max_depth,
                                                            int32_t* __restrict__ out_tokens,
                                                            int32_t* __restrict__ out_n,
                                                            int32_t* __restrict__ out_last) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int N = dm.K;  // nodes per tree (stored in K for the tree launch)
  constexpr int PER = kTreeMaxNodes / kTreeThreads;
  __shared__ int s_g[kTreeMaxNodes];
  __shared__ int s_par[kTreeMaxNodes];
  __shared__ int s_tok[kTreeMaxNodes];
  __shared__ uint32_t s_jump[2][kTreeMaxNodes];
  __shared__ int s_best[kTreeThreads / 64];
  // argmax of every node's row; parents and tokens
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + kTreeThreads * j;
    if (i >= N) break;
    const ChunkPart* p = ws.parts + ((size_t)b * N + i) * dm.nchunks;
    float best = p[0].vmax;
    int am = p[0].argmax;
    for (int c = 1; c < dm.nchunks; ++c) {
      const float v = p[c].vmax;
      if (v > best) {
        best = v;
        am = p[c].argmax;
      }
    }
    s_g[i] = am;
    s_par[i] = parent[(size_t)b * N + i];
    s_tok[i] = tokens[(size_t)b * N + i];
  }
  __syncthreads();
  // initial words: the root is a terminal; a node with a valid parent points at it with
  // distance 1 and ok = (its token is the parent's argmax); an invalid parent makes the node a
  // terminal that is not ok, and so every node below it
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + kTreeThreads * j;
    if (i >= N) break;
    uint32_t w;
    if (i == 0) {
      w = kJumpOk;
    } else {
      const int par = s_par[i];
      if (par >= 0 && par < i)
        w = (uint32_t)par | (1u << 11) | (s_tok[i] == s_g[par] ? kJumpOk : 0u);
      else
        w = (uint32_t)i;
    }
    s_jump[0][i] = w;
  }
  __syncthreads();
  int cur = 0;
  for (int span = 1; span < N; span <<= 1) {  // ceil(log2 N) rounds
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + kTreeThreads * j;
      if (i >= N) break;
      const uint32_t w = s_jump[cur][i];
      const uint32_t wa = s_jump[cur][w & kJumpA];
      const uint32_t d = ((w >> 11) & kJumpA) + ((wa >> 11) & kJumpA);
      s_jump[cur ^ 1][i] = (wa & kJumpA) | (d << 11) | (w & wa & kJumpOk);
    }
    __syncthreads();
    cur ^= 1;
  }
  // deepest accepted node, lowest index on ties: max of (depth, 2047 - index)
  int key = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + kTreeThreads * j;
    if (i >= N) break;
    const uint32_t w = s_jump[cur][i];
    const int d = (int)((w >> 11) & kJumpA);
    if ((w & kJumpOk) && d <= max_depth) key = max(key, (d << 11) | (2047 - i));
  }
  key = wave_reduce(key, [](int x, int y) { return x > y ? x : y; });
  if (lane_id() == 0) s_best[wave_id()] = key;
  __syncthreads();
  key = max(max(s_best[0], s_best[1]), max(s_best[2], s_best[3]));
  const int best = 2047 - (key & 2047);
  const int depth = key >> 11;
  int32_t* o = out_tokens + (size_t)b * (max_depth + 1);
  for (int j = depth + 1 + tid; j <= max_depth; j += kTreeThreads) o[j] = -1;
  if (tid == 0) {
    int i = best;
    for (int j = depth - 1; j >= 0; --j) {
      o[j] = s_tok[i];
      i = s_par[i];
    }
    o[depth] = s_g[best];
    out_n[b] = depth;
    if (out_last) out_last[b] = best;
  }
}

// ------------------------------------------------------------------------------------------
// Acceptance rate of every draft position (Leviathan blog, section 方法细节: the acceptance
// rate of one position is beta = 1 - D_LK(p, q) = sum_x min(p(x), q(x)), alpha = E(beta);
// with lenience l the accept test compares against q/l, so beta = sum_x min(p(x), q(x)/l)).
// One workgroup per position: greedy rows compare their argmaxes; two compact rows sum over
// the target's kept list in one wave; otherwise both full rows are streamed.
// ------------------------------------------------------------------------------------------
template <class E, bool VEC>
__global__ __launch_bounds__(kThreads) void k_beta(const E* __restrict__ tgt,
                                                   const E* __restrict__ drf, Dims dm, Samp sp,
                                                   Workspace ws, float* __restrict__ out_beta) {
  __shared__ RedScratch red;
  const int pos = blockIdx.x;
  const int b = pos / dm.K, k = pos - b * dm.K;
  const RowStat rt = ws.rstat[target_row(dm, b, k)];
  const RowStat rd = ws.rstat[draft_row(dm, b, k)];
  const float it = sp.inv_t;
  const double inv_l = 1.0 / (double)sp.lenience;
  if (rt.kind == kRowGreedy) {  // one-hot rows: min(p, q/l) = 1 at a shared argmax
    if (threadIdx.x == 0) out_beta[pos] = rt.argmax == rd.argmax ? 1.0f : 0.0f;
    return;
  }
  const E* drow = row_ptr(dm, tgt, drf, draft_row(dm, b, k));
  if (rt.kind == kRowCompact && rd.kind == kRowCompact) {
    if (wave_id() != 0) return;
    const uint2* kept = ws.kept + (size_t)target_row(dm, b, k) * kKeptCap;
    double acc = 0.0;
    for (int e = lane_id(); e < rt.nkept; e += 64) {
      const uint2 v = kept[e];
      const double q = (double)kept_exp(__uint_as_float(v.y), rt, it) / rt.S;
      const double p = (double)kept_exp(load_logit(drow, (int)v.x), rd, it) / rd.S;
      acc += p < q * inv_l ? p : q * inv_l;
    }
    acc = wave_reduce(acc, [](double a, double c) { return a + c; });
    if (lane_id() == 0) out_beta[pos] = (float)acc;
    return;
  }
  constexpr int EPV = Tr<E>::kEpv;
  const E* trow = row_ptr(dm, tgt, drf, target_row(dm, b, k));
  const int nvec = (dm.V + EPV - 1) / EPV;
  double acc = 0.0;
  for (int v = threadIdx.x; v < nvec; v += kThreads) {
    float zt[EPV], zd[EPV];
    load_vec_f<E, VEC>(trow, dm.V, v * EPV, zt);
    load_vec_f<E, VEC>(drow, dm.V, v * EPV, zd);
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const double q = (double)kept_exp(zt[e], rt, it) / rt.S * inv_l;
      const double p = (double)kept_exp(zd[e], rd, it) / rd.S;
      part += p < q ? p : q;
    }
    acc += part;
  }
  acc = block_sum_d(acc, red);
  if (threadIdx.x == 0) out_beta[pos] = (float)acc;
}

// Dense rows (no kept lists): one workgroup per (position, chunk) sums min(p, q/l) over the
// chunk into the chunk-partials array, which k_row has finished with; k_beta_merge adds the
// chunks of each position in order.
template <class E, bool VEC>
__global__ __launch_bounds__(kThreads) void k_beta_partial(const E* __restrict__ tgt,
                                                           const E* __restrict__ drf, Dims dm,
                                                           Samp sp, Workspace ws) {
  __shared__ RedScratch red;
  // one workgroup per (position, final chunk): the final draw's grain, so that few sequences
  // still fill the CUs
  const int pos = blockIdx.x / dm.nfchunks;
  const int c = blockIdx.x - pos * dm.nfchunks;
  const int b = pos / dm.K, k = pos - b * dm.K;
  const RowStat rt = ws.rstat[target_row(dm, b, k)];
  const RowStat rd = ws.rstat[draft_row(dm, b, k)];
  const float it = sp.inv_t;
  const double inv_l = 1.0 / (double)sp.lenience;
  constexpr int EPV = Tr<E>::kEpv;
  const E* trow = row_ptr(dm, tgt, drf, target_row(dm, b, k));
  const E* drow = row_ptr(dm, tgt, drf, draft_row(dm, b, k));
  const int e0 = c * dm.fchunk_elems;
  const int e1 = min(dm.V, e0 + dm.fchunk_elems);
  // fp32 per element with the normalisers folded into one factor per row, fp64 across vectors
  const float ft = (float)(inv_l / rt.S), fd = (float)(1.0 / rd.S);
  double acc = 0.0;
  for (int e = e0 + threadIdx.x * EPV; e < e1; e += kThreads * EPV) {
    float zt[EPV], zd[EPV];
    load_vec_f<E, VEC>(trow, dm.V, e, zt);
    load_vec_f<E, VEC>(drow, dm.V, e, zd);
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < EPV; ++j)
      part += fminf(kept_exp(zd[j], rd, it) * fd, kept_exp(zt[j], rt, it) * ft);
    acc += (double)part;
  }
  acc = block_sum_d(acc, red);
  if (threadIdx.x == 0) ws.bpart[(size_t)pos * dm.nfchunks + c] = acc;
}

// One wave per position: lanes take the chunks in a fixed stride, then a fixed-order wave sum.
__global__ __launch_bounds__(kThreads) void k_beta_merge(Dims dm, Workspace ws,
                                                         float* __restrict__ out_beta) {
  const int pos = blockIdx.x * (kThreads / 64) + wave_id();
  if (pos >= dm.B * dm.K) return;  // the whole wave
  double acc = 0.0;
  for (int c = lane_id(); c < dm.nfchunks; c += 64) acc += ws.bpart[(size_t)pos * dm.nfchunks + c];
  acc = wave_reduce(acc, [](double x, double y) { return x + y; });
  if (lane_id() == 0) out_beta[pos] = (float)acc;
}

// ------------------------------------------------------------------------------------------
// Launch helpers
// ------------------------------------------------------------------------------------------
// The final draw's two kernels at the grain Dims chose (see make_dims); LIST also draws the
// top-p sequences whose kept segments are complete.
template <class E, bool VEC, bool LIST>
void launch_final(const E* t, const E* d, const Dims& dm, const Samp& sp, const Workspace& ws,
                  const float* uni, int32_t* out_tokens, hipStream_t st) {
  const int G = LIST ? max(dm.nfchunks, dm.nchunks) : dm.nfchunks;
  const dim3 pgrid((unsigned)((size_t)dm.B * G));
  const bool partial = LIST || dm.nfchunks > 1;
  if (dm.fchunk_elems == dm.chunk_elems) {
    if (partial)
      hipLaunchKernelGGL((k_final_partial<E, VEC, kVecPerThread, LIST>), pgrid, dim3(kThreads), 0,
                         st, t, d, dm, sp, ws);
    hipLaunchKernelGGL((k_final_pick<E, VEC, kVecPerThread, LIST>), dim3(dm.B), dim3(kThreads), 0,
                       st, t, d, dm, sp, ws, uni, out_tokens);
  } else if (dm.fchunk_elems * 4 == dm.chunk_elems) {  // four vector rows per final chunk
    if (partial)
      hipLaunchKernelGGL((k_final_partial<E, VEC, 4, LIST>), pgrid, dim3(kThreads), 0, st, t, d,
                         dm, sp, ws);
    hipLaunchKernelGGL((k_final_pick<E, VEC, 4, LIST>), dim3(dm.B), dim3(kThreads), 0, st, t, d,
                       dm, sp, ws, uni, out_tokens);
  } else {  // one vector row per final chunk
    if (partial)
      hipLaunchKernelGGL((k_final_partial<E, VEC, 1, LIST>), pgrid, dim3(kThreads), 0, st, t, d,
                         dm, sp, ws);
    hipLaunchKernelGGL((k_final_pick<E, VEC, 1, LIST>), dim3(dm.B), dim3(kThreads), 0, st, t, d,
                       dm, sp, ws, uni, out_tokens);
  }
}

template <class E, bool VEC>
hipError_t launch_verify_t(const E* t, const E* d, const Dims& dm, const Samp& sp,
                           const int32_t* drafts, const float* uni, int32_t* out_tokens,
                           int32_t* out_n, float* out_a, float* out_q, float* out_p,
                           float* out_beta, bool rates_only, const Workspace& ws, hipStream_t st,
                           hipEvent_t* ev, int nev, const Workspace* presampled) {
  if (ev && nev >= 1) (void)hipEventRecord(ev[0], st);
  const unsigned grid_chunks = (unsigned)((size_t)dm.rows * dm.nchunks);
  const Outs o{drafts, uni, out_tokens, out_n, out_a, out_q, out_p};
  // rows of one chunk with nothing truncated: k_chunk's partials are the row statistics
  const bool row_is_chunk = dm.nchunks == 1 && !sp.greedy && !sp.topp_hist &&
                            !(sp.top_k > 0 && sp.top_k < dm.V) && !(sp.top_p < 1.0f);
  if (sp.compact) {
    // large k: the tile-0 threshold from 1024 group maxima (a kernel of its own)
    auto topk_row = sp.top_k > 64 ? k_topk_row<E, true> : k_topk_row<E, false>;
    if (presampled && dm.K > 0) {  // draft rows summarised by spec_sample: stream the targets only
      hipLaunchKernelGGL(k_take_draft_summaries, dim3(dm.B * dm.K), dim3(64), 0, st, dm,
                         *presampled, ws);
      hipLaunchKernelGGL(topk_row, dim3(dm.B * (dm.K + 1)), dim3(kThreads), 0, st, t, d, dm, sp,
                         ws, 1);
    } else {
      hipLaunchKernelGGL(topk_row, dim3(dm.rows), dim3(kThreads), 0, st, t, d, dm, sp, ws, 0);
    }
    if (ev && nev >= 2) (void)hipEventRecord(ev[1], st);
    if (out_beta) {  // acceptance rates from the row summaries (read-only for the steps below)
      hipLaunchKernelGGL((k_beta<E, VEC>), dim3(dm.B * dm.K), dim3(kThreads), 0, st, t, d, dm,
                         sp, ws, out_beta);
      if (rates_only) return hipGetLastError();
    }
    if (sp.mentor && dm.K > 0) {
      const int need_all = out_a != nullptr ? 1 : 0;
      hipLaunchKernelGGL((k_mentor<E>), dim3(dm.B * dm.K), dim3(64), 0, st, t, d, dm, sp, ws,
                         drafts, uni, need_all);
      hipLaunchKernelGGL((k_seq_compact<E, VEC, true>), dim3(dm.B), dim3(kThreads), 0, st, t, d,
                         dm, sp, ws, o);
    } else {
      hipLaunchKernelGGL((k_seq_compact<E, VEC, false>), dim3(dm.B), dim3(kThreads), 0, st, t, d,
                         dm, sp, ws, o);
    }
    if (ev && nev >= 3) (void)hipEventRecord(ev[2], st);
    return hipGetLastError();
  }
  // small problems: one launch, one workgroup per sequence holding all of its rows
  const bool dense_rows = !sp.greedy && !sp.topp_hist && !sp.generic_trunc && sp.top_k == 0 &&
                          !(sp.top_p < 1.0f) && !out_beta;
  const int R = dm.rows_per_seq;
  if (dense_rows && dm.draft_rows >= dm.K) {
    auto small = [&](auto kern, int L) {
      if (dm.V > kThreads * L || R > kSmallRegs / L) return false;
      hipLaunchKernelGGL(kern, dim3(dm.B), dim3(kThreads), 0, st, t, d, dm, sp, ws, o);
      if (ev && nev >= 2) (void)hipEventRecord(ev[1], st);
      if (ev && nev >= 3) (void)hipEventRecord(ev[2], st);
      return true;
    };
    if (small(k_small<E, 4>, 4) || small(k_small<E, 8>, 8) || small(k_small<E, 16>, 16))
      return hipGetLastError();
  }
  if (sp.greedy)
    hipLaunchKernelGGL((k_chunk_argmax<E>), dim3(grid_chunks), dim3(kThreads), 0, st, t, d, dm, sp,
                       ws);
  else if (sp.topp_hist)
    hipLaunchKernelGGL((k_chunk<E, true>), dim3(grid_chunks), dim3(kThreads), 0, st, t, d, dm,
                       sp, ws);
  else if (row_is_chunk)
    hipLaunchKernelGGL((k_chunk<E, false, true>), dim3(grid_chunks), dim3(kThreads), 0, st, t,
                       d, dm, sp, ws);
  else
    hipLaunchKernelGGL((k_chunk<E>), dim3(grid_chunks), dim3(kThreads), 0, st, t, d, dm, sp,
                       ws);
  if (ev && nev >= 2) (void)hipEventRecord(ev[1], st);
  if constexpr (sizeof(E) == 4) {
    if (sp.topp_hist)  // fp32 top-p: the bracket, the codes' candidates and the selection
      hipLaunchKernelGGL((k_topp_row<VEC>), dim3(dm.rows), dim3(kThreads), 0, st, t, d, dm, sp,
                         ws);
    else if (!row_is_chunk)
      hipLaunchKernelGGL((k_row<E, VEC>), dim3(dm.rows), dim3(kThreads), 0, st, t, d, dm, sp,
                         ws);
  } else {
    if (!row_is_chunk)
      hipLaunchKernelGGL((k_row<E, VEC>), dim3(dm.rows), dim3(kThreads), 0, st, t, d, dm, sp,
                         ws);
    if (sp.topp_hist) {
      hipLaunchKernelGGL((k_topp_cand<E>), dim3(grid_chunks), dim3(kThreads), 0, st, t, d, dm,
                         sp, ws);
      hipLaunchKernelGGL((k_topp_select<E, VEC>), dim3(dm.rows), dim3(kThreads), 0, st, t, d,
                         dm, sp, ws);
    }
  }
  if (out_beta) {  // acceptance rates
    if (sp.greedy) {
      hipLaunchKernelGGL((k_beta<E, VEC>), dim3(dm.B * dm.K), dim3(kThreads), 0, st, t, d, dm,
                         sp, ws, out_beta);
    } else {
      const int npos = dm.B * dm.K;
      hipLaunchKernelGGL((k_beta_partial<E, VEC>), dim3((unsigned)((size_t)npos * dm.nfchunks)),
                         dim3(kThreads), 0, st, t, d, dm, sp, ws);
      constexpr int kWaves = kThreads / 64;  // one wave per position
      hipLaunchKernelGGL(k_beta_merge, dim3((npos + kWaves - 1) / kWaves), dim3(kThreads), 0,
                         st, dm, ws, out_beta);
    }
    if (rates_only) return hipGetLastError();
  }
  hipLaunchKernelGGL((k_seq<E>), dim3(dm.B), dim3(kSeqThreads), 0, st, t, d, dm, sp, ws, o);
  if (!sp.greedy) {
    if (sp.topp_hist)  // each sequence drawn from its kept segments or, if incomplete, its rows
      launch_final<E, VEC, true>(t, d, dm, sp, ws, uni, out_tokens, st);
    else
      launch_final<E, VEC, false>(t, d, dm, sp, ws, uni, out_tokens, st);
  }
  if (ev && nev >= 3) (void)hipEventRecord(ev[2], st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const void* target, const void* draft, sv_dtype dt, const Dims& d,
                         const Samp& s, const int32_t* drafts, const float* uniforms,
                         int32_t* out_tokens, int32_t* out_n, float* out_a, float* out_q,
                         float* out_p, float* out_beta, bool rates_only, const Workspace& ws,
                         hipStream_t stream, hipEvent_t* events, int n_events,
                         const Workspace* presampled) {
  (void)hipGetLastError();  // clear a stale error so the status reflects these launches
  if (dt == SV_DTYPE_BF16) {
    auto t = static_cast<const uint16_t*>(target);
    auto dr = static_cast<const uint16_t*>(draft);
    if (d.vec)
      return launch_verify_t<uint16_t, true>(t, dr, d, s, drafts, uniforms, out_tokens, out_n,
                                             out_a, out_q, out_p, out_beta, rates_only, ws,
                                             stream, events, n_events, presampled);
    return launch_verify_t<uint16_t, false>(t, dr, d, s, drafts, uniforms, out_tokens, out_n,
                                            out_a, out_q, out_p, out_beta, rates_only, ws, stream,
                                            events, n_events, presampled);
  }
  auto t = static_cast<const float*>(target);
  auto dr = static_cast<const float*>(draft);
  if (d.vec)
    return launch_verify_t<float, true>(t, dr, d, s, drafts, uniforms, out_tokens, out_n, out_a,
                                        out_q, out_p, out_beta, rates_only, ws, stream, events,
                                        n_events, presampled);
  return launch_verify_t<float, false>(t, dr, d, s, drafts, uniforms, out_tokens, out_n, out_a,
                                       out_q, out_p, out_beta, rates_only, ws, stream, events,
                                       n_events, presampled);
}

hipError_t launch_tree(const void* target, sv_dtype dt, const Dims& d, const int32_t* parent,
                       const int32_t* tokens, int max_depth, int32_t* out_tokens,
                       int32_t* out_n, int32_t* out_last, const Workspace& ws,
                       hipStream_t stream, hipEvent_t* ev, int nev) {
  (void)hipGetLastError();
  if (ev && nev >= 1) (void)hipEventRecord(ev[0], stream);
  Samp sp{};
  sp.greedy = 1;
  const unsigned grid = (unsigned)((size_t)d.rows * d.nchunks);
  if (dt == SV_DTYPE_BF16) {
    auto t = static_cast<const uint16_t*>(target);
    hipLaunchKernelGGL((k_chunk_argmax<uint16_t>), dim3(grid), dim3(kThreads), 0, stream,
                       t, t, d, sp, ws);
  } else {
    auto t = static_cast<const float*>(target);
    hipLaunchKernelGGL((k_chunk_argmax<float>), dim3(grid), dim3(kThreads), 0, stream, t,
                       t, d, sp, ws);
  }
  if (ev && nev >= 2) (void)hipEventRecord(ev[1], stream);
  if (d.K <= 64)  // one wave per tree
    hipLaunchKernelGGL(k_tree_walk64, dim3(d.B), dim3(64), 0, stream, d, ws, parent, tokens,
                       max_depth, out_tokens, out_n, out_last);
  else
    hipLaunchKernelGGL(k_tree_walk, dim3(d.B), dim3(kTreeThreads), 0, stream, d, ws, parent,
                       tokens, max_depth, out_tokens, out_n, out_last);
  if (ev && nev >= 3) (void)hipEventRecord(ev[2], stream);
  return hipGetLastError();
}

}  // namespace sv
