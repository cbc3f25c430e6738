// 2:4 sparse x dense product on the gfx950 structured-sparse matrix cores
// (v_smfmac), with the per-token x per-channel rescale epilogue.
// Deep reading of arXiv 2610.28947 (introduction: one operand keeps two of
// every four along the accumulate axis; section 3.1: sparse W or sparse X);
// SlideSparse blog section 2.2 step 3; LLM Compressor W8A8 scales.
//
// C[r][c] = sum_k A[r][k] B[c][k] where A is the compressed operand (rows r)
// and B the dense one (rows c). side W: r = output channel n, c = token m.
// side X: r = token m, c = output channel n.
//
// gfx950 operand layout (16x16 instructions; measured on the hardware):
//   A lane l: row l%16, one 16-byte slice of compressed values covering 32
//     (8-bit) or 16 (16-bit) dense K positions, block (l/16) of the step, plus
//     a 32- or 16-bit index holding the 2:4 nibbles of exactly those groups;
//   B lane l: row l%16, two 16-byte slices at byte offsets 16*(l/16) and
//     64 + 16*(l/16) of the step's 128-byte K slice;
//   D lane l: rows 4*(l/16)+i (i = 0..3) of A, column l%16 of B.
// In bytes the two element widths are identical (a step is 64 compressed
// bytes of A and 128 bytes of B per row); only the index width differs.
//
// Tiling: 128 (A rows) x 128 (B rows) per workgroup of 4 waves (2 x 2), each
// wave 64 x 64 = 4 x 4 instructions; K tile = 2 steps (128 B of A values,
// 256 B of B, 32 or 16 B of metadata per row). A and B tiles are stored in
// LDS in lane order, so every fragment read is one contiguous 1 KB per wave.
// The next K tile is prefetched into registers while the current one is
// multiplied.
#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_store.h"

namespace ss {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v16bf __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128;
constexpr int A_TILE = BM * 128;   // bytes of A values per K tile
constexpr int B_TILE = BN * 256;   // bytes of B per K tile
constexpr int M_STRIDE = 48;       // LDS row stride of the metadata tile

// AB: 0 = int8, 1 = fp8 e4m3, 2 = bf16.  YT: 0 = bf16, 1 = f32, 2 = i32.
template <int AB> struct Mma;
template <> struct Mma<0> {
  using Acc = v4i;
  __device__ static Acc run(const uint4& a, const uint4& b0, const uint4& b1, Acc c, uint32_t idx) {
    v4i av = __builtin_bit_cast(v4i, a);
    v8i bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_smfmac_i32_16x16x128_i8(av, bv, c, (int)idx, 0, 0);
  }
};
template <> struct Mma<1> {
  using Acc = v4f;
  __device__ static Acc run(const uint4& a, const uint4& b0, const uint4& b1, Acc c, uint32_t idx) {
    v4i av = __builtin_bit_cast(v4i, a);
    v8i bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(av, bv, c, (int)idx, 0, 0);
  }
};
template <> struct Mma<2> {
  using Acc = v4f;
  __device__ static Acc run(const uint4& a, const uint4& b0, const uint4& b1, Acc c, uint32_t idx) {
    v8bf av = __builtin_bit_cast(v8bf, a);
    struct P { uint4 x, y; } p{b0, b1};
    v16bf bv = __builtin_bit_cast(v16bf, p);
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(av, bv, c, (int)idx, 0, 0);
  }
};


template <int AB, int YT, bool SIDE_X>
__global__ __launch_bounds__(256, 2) void spgemm_kernel(int64_t R, int64_t C, int64_t Kc,
                                                        const uint8_t* __restrict__ av, int64_t lda,  // bytes
                                                        const uint8_t* __restrict__ am, int64_t ldm,  // bytes
                                                        const uint8_t* __restrict__ bd, int64_t ldb,  // bytes
                                                        const float* __restrict__ sx, const float* __restrict__ sw,
                                                        void* __restrict__ Y, int64_t ldy, bool yvec) {
  constexpr int ES = (AB == 2) ? 2 : 1;          // element bytes
  constexpr int MB = (AB == 2) ? 16 : 32;        // metadata bytes per row per K tile
  using Acc = typename Mma<AB>::Acc;

  __shared__ __align__(16) uint8_t sA[A_TILE];
  __shared__ __align__(16) uint8_t sB[B_TILE];
  __shared__ __align__(16) uint8_t sM[BM * M_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t r0 = (int64_t)blockIdx.y * BM;
  const int64_t c0 = (int64_t)blockIdx.x * BN;
  const int64_t KT = Kc * ES / 256;  // K tiles

  // global -> register prefetch assignment
  uint4 pa[4], pb[8], pm;
  auto load_tile = [&](int64_t kt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int id = q * 256 + tid, row = id >> 3, c = id & 7;
      pa[q] = (r0 + row < R) ? *reinterpret_cast<const uint4*>(av + (r0 + row) * lda + kt * 128 + c * 16)
                             : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int id = q * 256 + tid, row = id >> 4, c = id & 15;
      pb[q] = (c0 + row < C) ? *reinterpret_cast<const uint4*>(bd + (c0 + row) * ldb + kt * 256 + c * 16)
                             : make_uint4(0, 0, 0, 0);
    }
    {
      const int row = (MB == 32) ? (tid >> 1) : tid, c = (MB == 32) ? (tid & 1) : 0;
      pm = (row < BM && r0 + row < R && (MB == 32 || tid < BM))
               ? *reinterpret_cast<const uint4*>(am + (r0 + row) * ldm + kt * MB + c * 16)
               : make_uint4(0x44444444u, 0x44444444u, 0x44444444u, 0x44444444u);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int id = q * 256 + tid, row = id >> 3, c = id & 7;
      const int i = row >> 4, r16 = row & 15, s = c >> 2, j = c & 3;
      *reinterpret_cast<uint4*>(sA + ((i * 2 + s) * 64 + j * 16 + r16) * 16) = pa[q];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int id = q * 256 + tid, row = id >> 4, c = id & 15;
      const int jt = row >> 4, r16 = row & 15, s = c >> 3, cc = c & 7, h = cc >> 2, j = cc & 3;
      *reinterpret_cast<uint4*>(sB + (((jt * 2 + s) * 2 + h) * 64 + j * 16 + r16) * 16) = pb[q];
    }
    if (MB == 32) {
      const int row = tid >> 1, c = tid & 1;
      *reinterpret_cast<uint4*>(sM + row * M_STRIDE + c * 16) = pm;
    } else if (tid < BM) {
      *reinterpret_cast<uint4*>(sM + tid * M_STRIDE) = pm;
    }
  };

  Acc acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  if (KT > 0) load_tile(0);
  for (int64_t kt = 0; kt < KT; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < KT) load_tile(kt + 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 fa[4];
      uint32_t fi[4];
      uint4 fb0[4], fb1[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = wm * 4 + t;
        fa[t] = *reinterpret_cast<const uint4*>(sA + ((i * 2 + s) * 64 + lane) * 16);
        const uint8_t* mp = sM + (i * 16 + (lane & 15)) * M_STRIDE;
        if (MB == 32) fi[t] = *reinterpret_cast<const uint32_t*>(mp + s * 16 + (lane >> 4) * 4);
        else fi[t] = *reinterpret_cast<const uint16_t*>(mp + s * 8 + (lane >> 4) * 2);
        const int jt = wn * 4 + t;
        fb0[t] = *reinterpret_cast<const uint4*>(sB + (((jt * 2 + s) * 2 + 0) * 64 + lane) * 16);
        fb1[t] = *reinterpret_cast<const uint4*>(sB + (((jt * 2 + s) * 2 + 1) * 64 + lane) * 16);
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) acc[ti][tj] = Mma<AB>::run(fa[ti], fb0[tj], fb1[tj], acc[ti][tj], fi[ti]);
    }
  }

  // epilogue: y = fl32(fl32(float(acc) * sx[m]) * sw[n])
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int64_t ar = r0 + (wm * 4 + ti) * 16 + 4 * (lane >> 4);  // 4 consecutive A rows
      const int64_t bc = c0 + (wn * 4 + tj) * 16 + (lane & 15);       // one B row
      if (bc >= C) continue;
      float y[4];
      int32_t yi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (YT == 2) {
          yi[q] = (int32_t)acc[ti][tj][q];
        } else {
          float f = (float)acc[ti][tj][q];
          const int64_t a = ar + q;
          const int64_t m = SIDE_X ? a : bc, nn = SIDE_X ? bc : a;
          if (a < R) {
            if (sx) f = __fmul_rn(f, sx[m]);
            if (sw) f = __fmul_rn(f, sw[nn]);
          }
          y[q] = f;
        }
      }
      if constexpr (!SIDE_X) {
        // Y[bc][ar .. ar+3]: 4 consecutive outputs of one token row
        if (yvec && ar + 3 < R) {
          if constexpr (YT == 0) {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + bc * ldy + ar) =
                make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
          } else if constexpr (YT == 1) {
            *reinterpret_cast<float4*>(static_cast<float*>(Y) + bc * ldy + ar) = make_float4(y[0], y[1], y[2], y[3]);
          } else {
            *reinterpret_cast<int4*>(static_cast<int32_t*>(Y) + bc * ldy + ar) = make_int4(yi[0], yi[1], yi[2], yi[3]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (ar + q >= R) break;
            if constexpr (YT == 0) static_cast<uint16_t*>(Y)[bc * ldy + ar + q] = f32_to_bf16(y[q]);
            else if constexpr (YT == 1) static_cast<float*>(Y)[bc * ldy + ar + q] = y[q];
            else static_cast<int32_t*>(Y)[bc * ldy + ar + q] = yi[q];
          }
        }
      } else {
        // Y[ar + q][bc]
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (ar + q >= R) break;
          if constexpr (YT == 0) static_cast<uint16_t*>(Y)[(ar + q) * ldy + bc] = f32_to_bf16(y[q]);
          else if constexpr (YT == 1) static_cast<float*>(Y)[(ar + q) * ldy + bc] = y[q];
          else static_cast<int32_t*>(Y)[(ar + q) * ldy + bc] = yi[q];
        }
      }
    }
  }
}


// ---------------------------------------------------------------------------
// 8-bit operands (int8, fp8): pipelined kernel.
//
// Each workgroup (8 waves, 4 x 2, wave tile 64 x 64) owns a 256 (sparse rows)
// x 128 (dense rows) output tile. The K loop runs in stages of two instruction
// steps (256 dense K): per sparse row 128 B of values (one cache line) and 32 B
// of metadata, per dense row 256 B (two lines). Operands move HBM/L2 -> LDS with
// global_load_lds_dwordx4 (no register round trip); each wave-load covers 8 rows
// x 128 B so every request is a full cache line (16 rows x 64 B halves the L2
// throughput on gfx950). Inside a line the 16-byte chunks are XOR-swizzled by
// row so the fragment reads are nearly free of LDS bank conflicts. Two LDS
// buffers: stage t+1 streams in while stage t is multiplied; within a stage the
// reads of step 1 are interleaved with the smfmacs of step 0.
// Rows past the matrix edge are clamped to the last row for loading; their
// results are never stored.
namespace pipe8 {

constexpr int BM = 256, BN = 128, WGM = 4, WGN = 2, NW = WGM * WGN;
constexpr int TI = BM / WGM / 16, TJ = BN / WGN / 16;  // 4 x 4 instructions per wave per step
constexpr int A_BYTES = BM * 128, M_BYTES = BM * 32, B_BYTES = BN * 256;
constexpr int STAGE = A_BYTES + M_BYTES + B_BYTES;     // 72 KB
constexpr int LDS = 2 * STAGE;                         // 144 KB
constexpr int NA = BM / 8, NMETA = BM / 32, NB = BN / 8 * 2;
constexpr int PA = NA / NW, PB = NB / NW;
static_assert(NA % NW == 0 && NB % NW == 0 && NMETA <= NW, "load split");
#define SS_LDS __attribute__((address_space(3)))

__device__ __forceinline__ int swz(int c, int r16) { return c ^ ((r16 >> 1) & 7); }

template <int AB, int YT, bool SIDE_X>
__global__ __launch_bounds__(64 * NW, 1) void spgemm8_kernel(int R, int C, int KT, const uint8_t* __restrict__ av, int lda,
                                                             const uint8_t* __restrict__ am, int ldm,
                                                             const uint8_t* __restrict__ bd, int ldb,
                                                             const float* __restrict__ sx, const float* __restrict__ sw,
                                                             void* __restrict__ Y, int ldy, int tiles_r, int tiles_c) {
  using Acc = typename Mma<AB>::Acc;
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // Tile order: the dispatcher deals workgroups to the 8 XCDs round-robin; give
  // each XCD a contiguous run of tiles, walked in groups of 4 sparse-row tiles,
  // so the tiles sharing operands also share an L2.
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  constexpr int GR = 4;
  const int group = bid / (GR * tiles_c);
  const int first_r = group * GR;
  const int gsize = min(tiles_r - first_r, GR);
  const int tr = first_r + (bid % (GR * tiles_c)) % gsize;
  const int tc = (bid % (GR * tiles_c)) / gsize;
  const int r0 = tr * BM, c0 = tc * BN;

  // per-lane source offsets of this wave's loads (stage 0)
  uint32_t offa[PA], offb[PB], offm = 0;
  const int r8 = lane >> 3, p = lane & 7;
#pragma unroll
  for (int q = 0; q < PA; ++q) {
    const int a = (wave + q * NW) * 8 + r8;
    offa[q] = (uint32_t)min(r0 + a, R - 1) * lda + swz(p, a & 15) * 16;
  }
#pragma unroll
  for (int q = 0; q < PB; ++q) {
    const int blk = wave + q * NW, b = (blk >> 1) * 8 + r8;
    offb[q] = (uint32_t)min(c0 + b, C - 1) * ldb + (blk & 1) * 128 + swz(p, b & 15) * 16;
  }
  if (wave < NMETA) offm = (uint32_t)min(r0 + wave * 32 + (lane >> 1), R - 1) * ldm + (lane & 1) * 16;

  auto issue = [&](int t) {
    SS_LDS uint8_t* base = (SS_LDS uint8_t*)smem + (t & 1) * STAGE;
#pragma unroll
    for (int q = 0; q < PA; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(av + offa[q] + t * 128), (SS_LDS void*)(base + (wave + q * NW) * 1024),
                                       16, 0, 0);
#pragma unroll
    for (int q = 0; q < PB; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(bd + offb[q] + t * 256),
                                       (SS_LDS void*)(base + A_BYTES + M_BYTES + (wave + q * NW) * 1024), 16, 0, 0);
    if (wave < NMETA)
      __builtin_amdgcn_global_load_lds((const void*)(am + offm + t * 32), (SS_LDS void*)(base + A_BYTES + wave * 1024), 16, 0, 0);
  };

  uint4 fa[2][TI], fb[2][TJ][2];
  uint32_t fi[2][TI];
  const int r16 = lane & 15, j = lane >> 4;
  auto read_frags = [&](int buf, int t, int s) {
    const uint8_t* st = smem + (t & 1) * STAGE;
#pragma unroll
    for (int u = 0; u < TI; ++u) {
      const int i = wm * TI + u, a = i * 16 + r16;
      fa[buf][u] = *reinterpret_cast<const uint4*>(st + (2 * i + (r16 >> 3)) * 1024 + (r16 & 7) * 128 + swz(s * 4 + j, r16) * 16);
      fi[buf][u] = *reinterpret_cast<const uint32_t*>(st + A_BYTES + (a >> 5) * 1024 + (a & 31) * 32 + s * 16 + j * 4);
    }
#pragma unroll
    for (int u = 0; u < TJ; ++u) {
      const int jt = wn * TJ + u;
      const uint8_t* bb = st + A_BYTES + M_BYTES + ((jt * 2 + (r16 >> 3)) * 2 + s) * 1024 + (r16 & 7) * 128;
      fb[buf][u][0] = *reinterpret_cast<const uint4*>(bb + swz(j, r16) * 16);
      fb[buf][u][1] = *reinterpret_cast<const uint4*>(bb + swz(4 + j, r16) * 16);
    }
  };
  Acc acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int u = 0; u < TJ; ++u) acc[i][u] = Acc{0, 0, 0, 0};
  auto mma = [&](int buf) {
#pragma unroll
    for (int u = 0; u < TJ; ++u)
#pragma unroll
      for (int i = 0; i < TI; ++i) acc[i][u] = Mma<AB>::run(fa[buf][i], fb[buf][u][0], fb[buf][u][1], acc[i][u], fi[buf][i]);
  };

  if (KT > 0) issue(0);
  for (int t = 0; t < KT; ++t) {
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0): this wave's loads of stage t landed
    __builtin_amdgcn_s_barrier();                         // everyone's landed; stage t-1 fully read
    if (t + 1 < KT) issue(t + 1);
    read_frags(0, t, 0);
    read_frags(1, t, 1);
    mma(0);
    mma(1);
    // step-0 reads, then step-0 smfmacs interleaved with step-1 reads, then the rest
    constexpr int RD = TI + TI / 2 + 2 * TJ;  // read instructions per step (metadata words pair up)
    constexpr int MF = TI * TJ;
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
#pragma unroll
    for (int q = 0; q < MF; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
  }

  // Epilogue: y = fl32(fl32(float(acc) * sx[m]) * sw[n]). All scales are loaded
  // up front (indices clamped; out-of-range results are never stored).
  float s_a[TI][4], s_b[TJ];
  const float* sa = SIDE_X ? sx : sw;  // scale indexed by sparse row
  const float* sb = SIDE_X ? sw : sx;  // scale indexed by dense row
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) s_a[i][q] = sa ? sa[min(r0 + (wm * TI + i) * 16 + 4 * j + q, R - 1)] : 1.0f;
#pragma unroll
  for (int u = 0; u < TJ; ++u) s_b[u] = sb ? sb[min(c0 + (wn * TJ + u) * 16 + r16, C - 1)] : 1.0f;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int u = 0; u < TJ; ++u) {
      const int ar = r0 + (wm * TI + i) * 16 + 4 * j;  // 4 consecutive sparse rows
      const int bc = c0 + (wn * TJ + u) * 16 + r16;    // one dense row
      if (bc >= C) continue;
      float y[4];
      int32_t yi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (YT == 2) {
          yi[q] = (int32_t)acc[i][u][q];
        } else {
          // the token scale is applied first, then the channel scale (an absent scale is 1: exact)
          const float s1 = SIDE_X ? s_a[i][q] : s_b[u], s2 = SIDE_X ? s_b[u] : s_a[i][q];
          y[q] = __fmul_rn(__fmul_rn((float)acc[i][u][q], s1), s2);
        }
      }
      store_out<YT, SIDE_X>(Y, ldy, ar, bc, R, y, yi);
    }
  }
}

}  // namespace pipe8

template <int AB, int YT>
static hipError_t launch_sg2(bool side_x, int64_t R, int64_t C, int64_t Kc, const uint8_t* av, int64_t lda,
                             const uint8_t* am, int64_t ldm, const uint8_t* bd, int64_t ldb, const float* sx,
                             const float* sw, void* Y, int64_t ldy, hipStream_t st) {
  const bool fits32 = (uint64_t)R * lda < (1ull << 32) && (uint64_t)R * ldm < (1ull << 32) &&
                      (uint64_t)C * ldb < (1ull << 32);
  if constexpr (AB != 2) {
   if (fits32) {
    // 8-bit pipelined kernel (32-bit operand offsets)
    const int tr = (int)((R + pipe8::BM - 1) / pipe8::BM), tc = (int)((C + pipe8::BN - 1) / pipe8::BN);
    const int KT = (int)(Kc / 256);
    auto kern = side_x ? pipe8::spgemm8_kernel<AB, YT, true> : pipe8::spgemm8_kernel<AB, YT, false>;
    const hipError_t e = lds_limit((const void*)kern, pipe8::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(tr * tc), dim3(64 * pipe8::NW), pipe8::LDS, st, (int)R, (int)C, KT, av, (int)lda, am,
                       (int)ldm, bd, (int)ldb, sx, sw, Y, (int)ldy, tr, tc);
    return hipGetLastError();
     }
  }
  dim3 grid((unsigned)((C + BN - 1) / BN), (unsigned)((R + BM - 1) / BM)), block(256);
  if (side_x)
    hipLaunchKernelGGL((spgemm_kernel<AB, YT, true>), grid, block, 0, st, R, C, Kc, av, lda, am, ldm, bd, ldb, sx, sw, Y, ldy, (ldy % 4) == 0);
  else
    hipLaunchKernelGGL((spgemm_kernel<AB, YT, false>), grid, block, 0, st, R, C, Kc, av, lda, am, ldm, bd, ldb, sx, sw, Y, ldy, (ldy % 4) == 0);
  return hipGetLastError();
}

hipError_t launch_spgemm(bool side_x, int ab, int yt, int64_t R, int64_t C, int64_t Kc, const void* av,
                         int64_t lda_bytes, const uint8_t* am, int64_t ldm, const void* bd, int64_t ldb_bytes,
                         const float* sx, const float* sw, void* Y, int64_t ldy, hipStream_t st) {
  const uint8_t* a = static_cast<const uint8_t*>(av);
  const uint8_t* b = static_cast<const uint8_t*>(bd);
#define SS_SG(AB_, YT_) return launch_sg2<AB_, YT_>(side_x, R, C, Kc, a, lda_bytes, am, ldm, b, ldb_bytes, sx, sw, Y, ldy, st)
  if (ab == 0) { if (yt == 0) SS_SG(0, 0); if (yt == 1) SS_SG(0, 1); SS_SG(0, 2); }
  if (ab == 1) { if (yt == 0) SS_SG(1, 0); SS_SG(1, 1); }
  if (yt == 0) SS_SG(2, 0);
  SS_SG(2, 1);
#undef SS_SG
}

}  // namespace ss
