// Offline SlideSparse weight preparation (SlideSparse article, sliding-window
// decomposition section and figure 2; SlideSparse blog sections 2.2-2.3):
// (2n-2):2n magnitude prune of each 2n-group, greedy assignment of the kept
// nonzeros to the n-1 stride-2 width-4 windows, per-channel quantisation and
// 2:4 compression of W' directly in K' order.
//
// Persistent workgroups, one weight row at a time. The row is staged in LDS with coalesced
// 16-byte loads (the absmax is taken on the way); thread i then owns groups
// i, i + 256, ... read back from LDS, prunes each, splits it into its n-1
// windows, quantises them and writes them into an LDS image of the output
// row, which leaves with 16-byte stores: row-major, or in the tiled layout of
// the product (16-byte lane chunks of 1 KB step blocks; index words gathered
// four steps at a time). Rows too long to stage use the register kernel
// (groups held in registers, or read twice when longer still).
#include "ss_device.h"
#include "ss_kernels.h"

#include <algorithm>

namespace ss {
namespace {

constexpr int kGPT = 8;                     // groups per thread held in registers (long-row kernel)
constexpr size_t kLdsMax = 160 * 1024;      // LDS of one CU

template <typename TIn> __device__ __forceinline__ float to_f32(TIn v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }

template <typename TIn> struct GroupIO;
template <> struct GroupIO<float> {
  // 2n floats at element offset 2n*g: 8-byte aligned for every n
  __device__ static void load(const float* row, int64_t g, int n, int64_t K, float* e) {
    const int64_t e0 = (int64_t)g * 2 * n;
    if (e0 + 2 * n <= K) {
      const float2* p = reinterpret_cast<const float2*>(row + e0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n) { const float2 v = p[i]; e[2 * i] = v.x; e[2 * i + 1] = v.y; }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < 2 * n) e[i] = (e0 + i < K) ? row[e0 + i] : 0.0f;
    }
  }
};
template <> struct GroupIO<uint16_t> {
  __device__ static void load(const uint16_t* row, int64_t g, int n, int64_t K, float* e) {
    const int64_t e0 = (int64_t)g * 2 * n;
    if (e0 + 2 * n <= K) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(row + e0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n) { const uint32_t v = p[i]; e[2 * i] = bf16_to_f32((uint16_t)(v & 0xFFFF)); e[2 * i + 1] = bf16_to_f32((uint16_t)(v >> 16)); }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < 2 * n) e[i] = (e0 + i < K) ? bf16_to_f32(row[e0 + i]) : 0.0f;
    }
  }
};

// Keep the 2n-2 largest magnitudes of the group (equal magnitudes keep the
// lower index): drop the smallest twice, where among equal magnitudes the
// higher index counts as smaller. Returns the bit mask of kept nonzeros.
template <int N>
__device__ __forceinline__ uint32_t keep_nonzero(const float* e) {
  constexpr int W = 2 * N;
  uint32_t key[W];
  uint32_t nonzero = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    key[i] = mag_key_f32(e[i]);
    nonzero |= (uint32_t)(key[i] != 0) << i;
  }
  uint32_t k1 = 0xFFFFFFFFu, b1 = 0;
#pragma unroll
  for (int i = 0; i < W; ++i)
    if (key[i] <= k1) { k1 = key[i]; b1 = i; }
  uint32_t k2 = 0xFFFFFFFFu, b2 = 0;
#pragma unroll
  for (int i = 0; i < W; ++i)
    if (i != (int)b1 && key[i] <= k2) { k2 = key[i]; b2 = i; }
  return nonzero & ~((1u << b1) | (1u << b2));
}

// The same mask, fast when there is no tie at the boundary: take the two
// smallest magnitudes v1 <= v2 as values (a running min and median), then the
// elements with |w| <= v2. Exactly two such elements are the dropped pair, and
// every other element is then larger than v2 >= 0, so nonzero. Three or more
// (equal magnitudes at v2, which includes three or more zeros) fall back to
// keep_nonzero.
template <int N>
__device__ __forceinline__ uint32_t keep_nonzero_fast(const float* e) {
  constexpr int W = 2 * N;
  float m1 = fminf(fabsf(e[0]), fabsf(e[1])), m2 = fmaxf(fabsf(e[0]), fabsf(e[1]));
#pragma unroll
  for (int i = 2; i < W; ++i) {
    const float a = fabsf(e[i]);
    m2 = __builtin_amdgcn_fmed3f(m1, m2, a);
    m1 = fminf(m1, a);
  }
  uint32_t le = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) le |= (fabsf(e[i]) <= m2) ? (1u << i) : 0u;
  if (__builtin_popcount(le) == 2) return ~le & ((1u << W) - 1);
  return keep_nonzero<N>(e);
}

// Greedy window assignment as a function of the kept-nonzero mask, for n = 3
// and n = 4 with 8-bit codes: `sel` holds the byte selectors (v_perm, over the
// group's codes packed 4 to a word; 0x0C gives a zero byte) of the two slots of
// windows 0 and 1, `aux` those of window 2 (bits 0-15) and the index nibbles of
// all windows (bits 16-27). Built at compile time from the same rule as
// emit_group.
template <int N> struct SlideTable { uint32_t sel[1 << (2 * N)], aux[1 << (2 * N)]; };
template <int N> constexpr SlideTable<N> make_slide_table() {
  SlideTable<N> t{};
  for (uint32_t nz = 0; nz < (1u << (2 * N)); ++nz) {
    uint32_t claimed = 0, sel = 0, aux = 0, mb = 0;
    for (int w = 0; w < N - 1; ++w) {
      uint32_t cand = nz & ~claimed & (0xFu << (2 * w));
      const uint32_t m1 = cand & (0u - cand);
      cand &= ~m1;
      const uint32_t m2 = cand & (0u - cand);
      const uint32_t mine = m1 | m2;
      claimed |= mine;
      const uint32_t own = mine >> (2 * w);
      uint32_t fill = own;
      for (int k = 0; k < 2; ++k) {
        int pc = 0;
        for (int b = 0; b < 4; ++b) pc += (int)((fill >> b) & 1u);
        if (pc < 2) fill |= (~fill) & (fill + 1);
      }
      int i0 = 0;
      while (!((fill >> i0) & 1u)) ++i0;
      int i1 = i0 + 1;
      while (!((fill >> i1) & 1u)) ++i1;
      const uint32_t s0 = ((own >> i0) & 1u) ? (uint32_t)(2 * w + i0) : 0x0Cu;
      const uint32_t s1 = ((own >> i1) & 1u) ? (uint32_t)(2 * w + i1) : 0x0Cu;
      if (w < 2) sel |= (s0 | (s1 << 8)) << (16 * w);
      else aux |= s0 | (s1 << 8);
      mb |= (uint32_t)(i0 | (i1 << 2)) << (4 * w);
    }
    if (N < 4) aux |= 0x0C0Cu;
    t.sel[nz] = sel;
    t.aux[nz] = aux | (mb << 16);
  }
  return t;
}
__constant__ SlideTable<3> kSlideTab3 = make_slide_table<3>();
__constant__ SlideTable<4> kSlideTab4 = make_slide_table<4>();

template <int N> constexpr bool kTablePath = (N == 3 || N == 4);

// Copy the table of pattern n into LDS (uint2 entries: sel, aux).
template <int N>
__device__ __forceinline__ void load_slide_table(uint2* tab) {
  if constexpr (N == 3) {
    for (int i = threadIdx.x; i < 64; i += kBlock) tab[i] = make_uint2(kSlideTab3.sel[i], kSlideTab3.aux[i]);
  } else if constexpr (N == 4) {
    for (int i = threadIdx.x; i < 256; i += kBlock) tab[i] = make_uint2(kSlideTab4.sel[i], kSlideTab4.aux[i]);
  }
}

// 8-bit code of one value with the row's inv (as Quant::code): INT8 rounds by
// adding 1.5 * 2^23, which leaves rint(t) in the low mantissa bits (t is
// clamped to +-127 first; both are integers, so clamping before or after the
// rounding is the same). FP8 uses the conversion unit.
template <int OUT>
__device__ __forceinline__ uint32_t code_bits(float v, float inv) {
  const float t = __fmul_rn(v, inv);
  if constexpr (OUT == 1) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(t, -448.0f, 448.0f), 0.0f, 0, false) & 0xFFu;
  } else {
    return __float_as_uint(__builtin_amdgcn_fmed3f(t, -127.0f, 127.0f) + 12582912.0f) & 0xFFu;
  }
}

// Table path (n = 3, 4; 8-bit codes): codes of all 2n elements, two v_perm for
// the slot bytes, one or two LDS ORs for the index nibbles. Slots that do not
// own a nonzero select a zero byte, so a zero row needs no special case.
template <int N, int OUT>
__device__ __forceinline__ void emit_group_tab(const float* e, int g, float inv, const uint2* tab, uint8_t* lv,
                                               uint32_t* lm) {
  const uint32_t nz = keep_nonzero_fast<N>(e);
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 2 * N; ++i) c[i >> 2] |= code_bits<OUT>(e[i], inv) << (8 * (i & 3));
  const uint2 en = tab[nz];
  const uint32_t v01 = __builtin_amdgcn_perm(c[1], c[0], en.x);
  constexpr int B = 2 * (N - 1);  // value bytes per group
  if constexpr (N == 3) {
    reinterpret_cast<uint32_t*>(lv)[g] = v01;
  } else {
    const uint32_t v2 = __builtin_amdgcn_perm(c[1], c[0], (en.y & 0xFFFFu) | 0x0C0C0000u);
    uint16_t* p = reinterpret_cast<uint16_t*>(lv + B * g);
    p[0] = (uint16_t)v01;
    p[1] = (uint16_t)(v01 >> 16);
    p[2] = (uint16_t)v2;
  }
  constexpr int MB = 4 * (N - 1);  // index bits per group
  const uint32_t mb = en.y >> 16;
  const int bit = MB * g, sh = bit & 31;
  atomicOr(&lm[bit >> 5], mb << sh);
  if (sh > 32 - MB) atomicOr(&lm[(bit >> 5) + 1], mb >> (32 - sh));
}

// Emit the n-1 windows of one group into the LDS row image: values (ES bytes
// each) at window slot 2t, 2t+1 and the nibble of window t into metadata word t/8.
template <int N, int OUT>
__device__ __forceinline__ void emit_group(const float* e, int64_t g, bool zero_row, float inv, uint8_t* lv, uint32_t* lm) {
  const uint32_t nz = keep_nonzero_fast<N>(e);
  uint32_t claimed = 0;
#pragma unroll
  for (int w = 0; w < N - 1; ++w) {
    // window w takes the unassigned nonzeros of positions 2w..2w+3, lowest first, up to two
    uint32_t cand = nz & ~claimed & (0xFu << (2 * w));
    const uint32_t m1 = cand & (0u - cand);
    cand &= ~m1;
    const uint32_t m2 = cand & (0u - cand);
    const uint32_t mine = m1 | m2;
    claimed |= mine;
    const uint32_t own = mine >> (2 * w);
    uint32_t fill = own;  // slots: owned positions, then the lowest free ones
    if (__builtin_popcount(fill) < 2) fill |= (~fill) & (fill + 1);
    if (__builtin_popcount(fill) < 2) fill |= (~fill) & (fill + 1);
    const uint32_t i0 = __builtin_ctz(fill), i1 = __builtin_ctz(fill & (fill - 1));
    // select with compile-time indices (a runtime index would put e[] in scratch memory)
    const float c0 = e[2 * w], c1 = e[2 * w + 1], c2 = e[2 * w + 2], c3 = e[2 * w + 3];
    const float x0 = i0 == 0 ? c0 : i0 == 1 ? c1 : i0 == 2 ? c2 : c3;
    const float x1 = i1 == 1 ? c1 : i1 == 2 ? c2 : c3;  // i1 > i0 >= 0
    const float v0 = (own >> i0 & 1) ? x0 : 0.0f;
    const float v1 = (own >> i1 & 1) ? x1 : 0.0f;
    const int64_t t = g * (N - 1) + w;
    if constexpr (OUT == 2) {
      reinterpret_cast<uint32_t*>(lv)[t] = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
    } else {
      const uint32_t q0 = zero_row ? 0u : (uint32_t)Quant<OUT == 1>::code(v0, inv);
      const uint32_t q1 = zero_row ? 0u : (uint32_t)Quant<OUT == 1>::code(v1, inv);
      reinterpret_cast<uint16_t*>(lv)[t] = (uint16_t)(q0 | (q1 << 8));
    }
    atomicOr(&lm[t >> 3], (i0 | (i1 << 2)) << (4 * (t & 7)));
  }
}

// Padding windows (K' rounded up to Kc): zero values, positions (0, 1).
template <int OUT>
__device__ __forceinline__ void emit_padding(int64_t t0, int64_t Kc, uint8_t* lv, uint32_t* lm) {
  for (int64_t t = t0 + threadIdx.x; t < Kc / 4; t += kBlock) {
    if constexpr (OUT == 2) reinterpret_cast<uint32_t*>(lv)[t] = 0;
    else reinterpret_cast<uint16_t*>(lv)[t] = 0;
    atomicOr(&lm[t >> 3], 0x4u << (4 * (t & 7)));
  }
}

// Store the finished LDS image of one output row (after a barrier).
// Row-major: vals + row * ldv_bytes, meta + row * ldm.
// Tiled (k_spgemm_tiled.hip layout; ldv_bytes = padded step count KSP): a step
// is 64 value bytes per row; chunk q (16 bytes) of the row is lane chunk q % 4
// of step q / 4, at 16 * (row % 16 + 16 * (q % 4)) in that step's 1 KB block of
// row block row / 16. Index words: 8-bit values have one 32-bit word per chunk,
// and the words of steps 4g..4g+3 of one lane chunk form 16 bytes of the 1 KB
// block g; bf16 values have 16 bits per chunk, 8 bytes per lane chunk in a
// 512-byte block. Steps past the data are padding (zero values, index 0x4).
template <int OUT, bool TILED>
__device__ __forceinline__ void store_image(const uint8_t* lv, const uint32_t* lm, int64_t row, int64_t Kc,
                                            uint8_t* __restrict__ vals, int64_t ldv_bytes, uint8_t* __restrict__ meta,
                                            int64_t ldm) {
  constexpr int ES = (OUT == 2) ? 2 : 1;
  const int64_t nchunk = Kc / 2 * ES / 16;
  if constexpr (!TILED) {
    uint8_t* vr = vals + row * ldv_bytes;
    uint8_t* mr = meta + row * ldm;
    for (int64_t c = threadIdx.x; c < nchunk; c += kBlock)
      reinterpret_cast<uint4*>(vr)[c] = reinterpret_cast<const uint4*>(lv)[c];
    for (int64_t c = threadIdx.x; c < Kc / 8 / 16; c += kBlock)
      reinterpret_cast<uint4*>(mr)[c] = reinterpret_cast<const uint4*>(lm)[c];
  } else {
    const int64_t KSP = ldv_bytes, KS4 = KSP / 4, rb = row >> 4;
    const int r = (int)(row & 15);
    for (int64_t q = threadIdx.x; q < KSP * 4; q += kBlock) {
      const int64_t s = q >> 2;
      const int lane = r + 16 * (int)(q & 3);
      const uint4 v = q < nchunk ? reinterpret_cast<const uint4*>(lv)[q] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(vals + (rb * KSP + s) * 1024 + 16 * lane) = v;
    }
    for (int64_t p = threadIdx.x; p < KS4 * 4; p += kBlock) {
      const int64_t g = p >> 2;
      const int c = (int)(p & 3), lane = r + 16 * c;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t q = 4 * (4 * g + j) + c;  // chunk of step 4g + j
        if constexpr (OUT == 2) w[j] = q < nchunk ? reinterpret_cast<const uint16_t*>(lm)[q] : 0x4444u;
        else w[j] = q < nchunk ? lm[q] : 0x44444444u;
      }
      if constexpr (OUT == 2)
        *reinterpret_cast<uint2*>(meta + (rb * KS4 + g) * 512 + 8 * lane) =
            make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
      else
        *reinterpret_cast<uint4*>(meta + (rb * KS4 + g) * 1024 + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Rows that fit in LDS. Dynamic LDS: [row, zero-padded to G * 2n elements, rounded
// to 16 bytes][values Kc/2 * ES][metadata Kc/8]. Persistent: iteration i of a
// workgroup takes row blockIdx.x + i * gridDim.x (TILED: in xcd_row order over the
// rows up to the next multiple of 16, those past `rows` written as zero rows).
// Each row is loaded when it is staged (four 16-byte loads in flight per
// thread); eight waves per SIMD (n <= 4) overlap one workgroup's loads with another's
// pruning. (A one-row-ahead register prefetch needed 86 VGPRs, five waves per
// SIMD, and measured 11% slower.)
template <typename TIn, int N, int OUT, bool TILED>
__global__ __launch_bounds__(kBlock, N <= 4 ? 8 : 4) void slide_lds_kernel(const TIn* __restrict__ W, int64_t ldw, int rows, int K,
                                                           uint8_t* __restrict__ vals, int64_t ldv_bytes,
                                                           uint8_t* __restrict__ meta, int64_t ldm, int Kc,
                                                           float* __restrict__ scale) {
  constexpr int ES = (OUT == 2) ? 2 : 1;
  constexpr int EPU = 16 / (int)sizeof(TIn);      // elements per 16-byte unit
  constexpr int GB = 2 * N * (int)sizeof(TIn);    // bytes per group
  constexpr bool TAB = kTablePath<N> && OUT != 2;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float red[kBlock / 64];
  __shared__ uint2 tab[TAB ? (1 << (2 * N)) : 1];
  const int G = (K + 2 * N - 1) / (2 * N);
  const int xbytes = (G * GB + 15) & ~15;
  TIn* lx = reinterpret_cast<TIn*>(lds);
  uint8_t* lv = lds + xbytes;
  uint32_t* lm = reinterpret_cast<uint32_t*>(lv + Kc / 2 * ES);
  const int tid = threadIdx.x;
  const int nrows = TILED ? (rows + 15) / 16 * 16 : rows;
  const int nfull = K / EPU;  // whole 16-byte units of a row
  auto row_of = [&](int it) { return TILED ? xcd_row(it, nrows) : it; };
  if constexpr (TAB) load_slide_table<N>(tab);  // published by the first barrier below

  for (int it = blockIdx.x; it < nrows; it += gridDim.x) {
    const int row = row_of(it);
    const bool live = row < rows;
    const TIn* wr = W + (int64_t)(live ? row : 0) * ldw;
    float amax = 0.0f;
    auto stage = [&](const uint4& v, int i) {
      reinterpret_cast<uint4*>(lx)[i] = v;
      const TIn* t = reinterpret_cast<const TIn*>(&v);
#pragma unroll
      for (int k = 0; k < EPU; ++k) amax = fmaxf(amax, fabsf(to_f32<TIn>(t[k])));
    };
    for (int i0 = 0; i0 < nfull; i0 += 4 * kBlock) {  // four loads in flight per thread (zeros past `rows`)
      uint4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * kBlock + tid;
        v[j] = (i < nfull && live) ? reinterpret_cast<const uint4*>(wr)[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * kBlock + tid;
        if (i < nfull) stage(v[j], i);
      }
    }
    // ragged end of the row and the zero padding of the last group
    for (int e = nfull * EPU + tid; e < G * 2 * N; e += kBlock) {
      const TIn v = (live && e < K) ? wr[e] : (TIn)0;
      lx[e] = v;
      amax = fmaxf(amax, fabsf(to_f32<TIn>(v)));
    }
    for (int i = tid; i < Kc / 32; i += kBlock) lm[i] = 0;
    bool zero_row = false;
    float inv = 0.0f;
    if constexpr (OUT != 2) {
      amax = block_max(amax, red);  // also publishes the staged row and the metadata clear
      constexpr float Q = (OUT == 1) ? 448.0f : 127.0f;
      zero_row = (amax == 0.0f);
      inv = zero_row ? 0.0f : Q / amax;
      if (tid == 0 && live) scale[row] = zero_row ? 0.0f : amax / Q;
    } else {
      lds_barrier();
    }
    for (int g = tid; g < G; g += kBlock) {
      float e[2 * N];
      const uint8_t* src = lds + g * GB;
      if constexpr (GB % 16 == 0) {
        // whole 16-byte LDS reads (ds_read_b128): lanes 32 or 64 bytes apart conflict at most 2-way
        typedef uint32_t v4u __attribute__((ext_vector_type(4)));
        const v4u* s4 = reinterpret_cast<const v4u*>(lds) + g * (GB / 16);
#pragma unroll
        for (int j = 0; j < GB / 16; ++j) {
          const v4u u = __builtin_nontemporal_load(s4 + j);
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int k = 0; k < EPU; ++k) {
            if constexpr (sizeof(TIn) == 4) e[j * EPU + k] = __uint_as_float(w[k]);
            else e[j * EPU + k] = bf16_to_f32((uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu)));
          }
        }
      } else if constexpr (GB % 8 == 0) {
        constexpr int E8 = 8 / (int)sizeof(TIn);
        const uint2* s2 = reinterpret_cast<const uint2*>(lds) + g * (GB / 8);
#pragma unroll
        for (int j = 0; j < GB / 8; ++j) {
          const uint2 u = s2[j];
          const uint32_t w[2] = {u.x, u.y};
#pragma unroll
          for (int k = 0; k < E8; ++k) {
            if constexpr (sizeof(TIn) == 4) e[j * E8 + k] = __uint_as_float(w[k]);
            else e[j * E8 + k] = bf16_to_f32((uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu)));
          }
        }
      } else {
        constexpr int E4 = 4 / (int)sizeof(TIn);
#pragma unroll
        for (int j = 0; j < GB / 4; ++j) {
          const uint32_t u = reinterpret_cast<const uint32_t*>(src)[j];
          const TIn* t = reinterpret_cast<const TIn*>(&u);
#pragma unroll
          for (int k = 0; k < E4; ++k) e[j * E4 + k] = to_f32<TIn>(t[k]);
        }
      }
      if constexpr (TAB) emit_group_tab<N, OUT>(e, g, inv, tab, lv, lm);
      else emit_group<N, OUT>(e, g, zero_row, inv, lv, lm);
    }
    emit_padding<OUT>((int64_t)G * (N - 1), Kc, lv, lm);
    lds_barrier();
    store_image<OUT, TILED>(lv, lm, row, Kc, vals, ldv_bytes, meta, ldm);
    lds_barrier();  // the next row overwrites the LDS image
  }
}

// Rows too long for LDS staging. Dynamic LDS: [values Kc/2 * ES][metadata Kc/8].
// Rows whose groups fit in the register budget (G <= 256 * kGPT) are read once;
// longer rows are read twice (the second pass mostly from cache). TILED as in
// slide_lds_kernel.
template <typename TIn, int N, int OUT, bool TILED>
__global__ __launch_bounds__(kBlock) void slide_kernel(const TIn* __restrict__ W, int64_t ldw, int64_t rows, int64_t K,
                                                       uint8_t* __restrict__ vals, int64_t ldv_bytes,
                                                       uint8_t* __restrict__ meta, int64_t ldm, int64_t Kc,
                                                       float* __restrict__ scale) {
  constexpr int ES = (OUT == 2) ? 2 : 1;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float red[kBlock / 64];
  uint8_t* lv = lds;
  uint32_t* lm = reinterpret_cast<uint32_t*>(lds + Kc / 2 * ES);
  const int64_t row = TILED ? xcd_row(blockIdx.x, gridDim.x) : blockIdx.x;
  const bool live = row < rows;
  const TIn* wr = W + (live ? row : 0) * ldw;
  const int tid = threadIdx.x;
  const int64_t G = live ? (K + 2 * N - 1) / (2 * N) : 0;
  const bool in_regs = G <= (int64_t)kBlock * kGPT;

  for (int64_t i = tid; i < Kc / 32; i += kBlock) lm[i] = 0;

  float e[kGPT][16];
  float amax = 0.0f;
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kGPT; ++q) {
      const int64_t g = tid + (int64_t)q * kBlock;
      if (g < G) {
        GroupIO<TIn>::load(wr, g, N, K, e[q]);
#pragma unroll
        for (int i = 0; i < 2 * N; ++i) amax = fmaxf(amax, fabsf(e[q][i]));
      }
    }
  } else {
    for (int64_t g = tid; g < G; g += kBlock) {
      float t[16];
      GroupIO<TIn>::load(wr, g, N, K, t);
#pragma unroll
      for (int i = 0; i < 2 * N; ++i) amax = fmaxf(amax, fabsf(t[i]));
    }
  }
  bool zero_row = false;
  float inv = 0.0f;
  if constexpr (OUT != 2) {
    amax = block_max(amax, red);  // also orders the metadata clear before the ORs below
    constexpr float Q = (OUT == 1) ? 448.0f : 127.0f;
    zero_row = (amax == 0.0f);
    inv = zero_row ? 0.0f : Q / amax;
    if (tid == 0 && live) scale[row] = zero_row ? 0.0f : amax / Q;
  } else {
    lds_barrier();
  }
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kGPT; ++q) {
      const int64_t g = tid + (int64_t)q * kBlock;
      if (g < G) emit_group<N, OUT>(e[q], g, zero_row, inv, lv, lm);
    }
  } else {
    for (int64_t g = tid; g < G; g += kBlock) {
      float t[16];
      GroupIO<TIn>::load(wr, g, N, K, t);
      emit_group<N, OUT>(t, g, zero_row, inv, lv, lm);
    }
  }
  emit_padding<OUT>(G * (N - 1), Kc, lv, lm);
  lds_barrier();
  store_image<OUT, TILED>(lv, lm, row, Kc, vals, ldv_bytes, meta, ldm);
}

template <typename TIn, int N, int OUT, bool TILED>
hipError_t launch_one(const TIn* W, int64_t ldw, int64_t rows, int64_t K, uint8_t* v, int64_t ldv_bytes, uint8_t* meta,
                      int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  constexpr int ES = (OUT == 2) ? 2 : 1;
  const int64_t nrows = TILED ? (rows + 15) / 16 * 16 : rows;
  const int64_t G = (K + 2 * N - 1) / (2 * N);
  const size_t image = (size_t)Kc / 2 * ES + (size_t)Kc / 8;
  const size_t staged = (((size_t)G * 2 * N * sizeof(TIn) + 15) & ~(size_t)15) + image;
  // the staged kernel also holds up to 2 KB of static LDS (reduction slots, window table)
  const bool small = staged + 4096 <= kLdsMax && K < (1 << 30) && Kc < (1 << 30) && rows < (1 << 30);
  if (!small) {
    const void* fn = (const void*)slide_kernel<TIn, N, OUT, TILED>;
    if (image > 64 * 1024) {
      const hipError_t e = lds_limit(fn, (int)image);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((slide_kernel<TIn, N, OUT, TILED>), dim3((unsigned)nrows), dim3(kBlock), image, st, W, ldw, rows,
                       K, v, ldv_bytes, meta, ldm, Kc, scale);
    return hipGetLastError();
  }
  // persistent grid: the workgroups that are resident at once (registers and LDS), at most 8
  // per CU; a multiple of 8 when it is smaller than the row count (xcd_row order)
  auto go = [&](auto kern) -> hipError_t {
    if (staged > 64 * 1024) {
      const hipError_t e = lds_limit((const void*)kern, (int)staged);
      if (e != hipSuccess) return e;
    }
    int per_cu = 0;
    per_cu = occupancy_p((const void*)kern, kBlock, staged);
    per_cu = std::min(per_cu, 8);
    const unsigned grid = (unsigned)std::min<int64_t>(nrows, (int64_t)num_cus_p() * per_cu);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), staged, st, W, ldw, (int)rows, (int)K, v, ldv_bytes, meta, ldm,
                       (int)Kc, scale);
    return hipGetLastError();
  };
  return go(slide_lds_kernel<TIn, N, OUT, TILED>);
}

template <typename TIn, int N, bool TILED>
hipError_t launch_n(int out, const TIn* W, int64_t ldw, int64_t rows, int64_t K, void* vals, int64_t ldv_bytes,
                    uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  uint8_t* v = static_cast<uint8_t*>(vals);
  switch (out) {
    case 0: return launch_one<TIn, N, 0, TILED>(W, ldw, rows, K, v, ldv_bytes, meta, ldm, Kc, scale, st);
    case 1: return launch_one<TIn, N, 1, TILED>(W, ldw, rows, K, v, ldv_bytes, meta, ldm, Kc, scale, st);
    default: return launch_one<TIn, N, 2, TILED>(W, ldw, rows, K, v, ldv_bytes, meta, ldm, Kc, scale, st);
  }
}

template <typename TIn, bool TILED>
hipError_t launch_sl(int out, const TIn* W, int64_t ldw, int64_t rows, int64_t K, int n, void* vals, int64_t ldv_bytes,
                     uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  switch (n) {
    case 2: return launch_n<TIn, 2, TILED>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 3: return launch_n<TIn, 3, TILED>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 4: return launch_n<TIn, 4, TILED>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 5: return launch_n<TIn, 5, TILED>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 6: return launch_n<TIn, 6, TILED>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    case 7: return launch_n<TIn, 7, TILED>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
    default: return launch_n<TIn, 8, TILED>(out, W, ldw, rows, K, vals, ldv_bytes, meta, ldm, Kc, scale, st);
  }
}

}  // namespace

hipError_t launch_slide(bool in_bf16, int out, const void* W, int64_t ldw, int64_t rows, int64_t K, int n, void* vals,
                        int64_t ldv_bytes, uint8_t* meta, int64_t ldm, int64_t Kc, float* scale, hipStream_t st) {
  if (in_bf16)
    return launch_sl<uint16_t, false>(out, static_cast<const uint16_t*>(W), ldw, rows, K, n, vals, ldv_bytes, meta, ldm,
                                      Kc, scale, st);
  return launch_sl<float, false>(out, static_cast<const float*>(W), ldw, rows, K, n, vals, ldv_bytes, meta, ldm, Kc,
                                 scale, st);
}

hipError_t launch_slide_tiled(bool in_bf16, int out, const void* W, int64_t ldw, int64_t rows, int64_t K, int n,
                              int64_t Kc, void* tv, uint8_t* tm, float* scale, hipStream_t st) {
  // n = 2 is the 2:4 prune: the unit kernel of k_prune.hip writes the same bytes without staging
  if (n == 2 && K < (1 << 30) && rows < (1 << 30))
    return launch_prune24_tiled(in_bf16, out, W, ldw, rows, K, Kc, tv, tm, scale, st);
  const int64_t KS = Kc * (out == 2 ? 2 : 1) / 128, KSP = (KS + 3) / 4 * 4;
  if (in_bf16)
    return launch_sl<uint16_t, true>(out, static_cast<const uint16_t*>(W), ldw, rows, K, n, tv, KSP, tm, 0, Kc, scale,
                                     st);
  return launch_sl<float, true>(out, static_cast<const float*>(W), ldw, rows, K, n, tv, KSP, tm, 0, Kc, scale, st);
}

}  // namespace ss
