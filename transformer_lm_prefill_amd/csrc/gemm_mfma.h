// 16-bit MFMA GEMM for the layer's projections: C = A · B^T with A [M, K] activations and
// B [N, K] weights in torch nn.Linear layout, fp32 accumulation on the gfx950 32x32x16 MFMA.
//
// Operand formats: A and the MFMA run in one 16-bit format (fp16 or bf16). B is stored in
// that format, or in bf16 while A is fp16: then B is converted to fp16 between LDS and the
// MFMA (exact for |w| in [2^-17, 65504]).
//
// Uses (hf2q 0.1.1, qwen3vl_text/forward.rs, module doc; cortiq-engine 0.8.21, qwen3te.rs,
// `encode_with_images`):
//   QKV      EPI_STORE_16, B rows drawn from Wq, Wk, Wv in turn (one launch for all three)
//   o-proj   EPI_STORE_F32 with the residual: y1 = x + o Wo^T
//   gate/up  EPI_SWIGLU_16: a = silu(yn Wg^T) * (yn Wu^T), the two products in one tile
//   down     EPI_STORE_F32 with the residual: y2 = y1 + a Wd^T
//
// Main kernel (gemm_d2l_kernel), tiled for gfx950 (256 CUs in 8 XCDs, 160 KiB LDS per CU):
//   workgroup tile 256 x BN (BN = 256, 192 or 128), 8 waves (two per SIMD, so one wave's LDS
//   and memory waits overlap the other's MFMAs), each wave a (256/WM) x (BN/WN) block of
//   32x32 MFMA tiles with fp32 accumulators;
//   tiles go from global memory straight into LDS (direct-to-LDS buffer loads, no staging
//   registers) through a 4-stage ring of 32-wide K steps, each requested three steps before
//   its MFMAs, one barrier per step;
//   MFMA operand fragments are read from LDS one 16-wide K sub-step ahead of their MFMAs;
//   16-byte LDS chunks XOR-permuted by row, so the fragment reads are free of bank conflicts
//   (rocprofv3 SQ_LDS_BANK_CONFLICT reads 0);
//   workgroup ids remapped so each XCD (ids congruent mod 8) owns a compact band of tiles
//   sharing A rows and B columns in its own L2;
//   for fp32 outputs the accumulators hold C^T blocks, so the residual epilogue moves 16-byte
//   runs of one row.
#pragma once

#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "kernels.h"

// LDS ring depth of the direct-to-LDS kernel (stages of 32-wide K steps; tiles that would not
// fit in 160 KiB use 4)
#ifndef Q3_GEMM_STAGES
#define Q3_GEMM_STAGES 4
#endif
// Where bf16 weights become fp16 in the direct-to-LDS kernel: 2: always in LDS, once per
// workgroup, by the thread whose load brought them (after its own wait, before the barrier
// that publishes the stage); 0: always per fragment, by every wave after its read; 1: in LDS
// for tiles whose B fragments are read by four or more waves, per fragment otherwise.
// 3: tiles whose B fragments four or more waves read (QKV) stage B through registers (global
// load, one conversion per element, LDS store), per fragment otherwise. Measured at the 8B
// shape: 3 is best (QKV 8% faster than 0, same bits); 1 and 2 add a read and a write of the B
// tile to the LDS traffic that bounds the kernel (QKV 5% slower than 0); staging the
// two-wave-shared tiles of o-proj / down too gains at most 1%, and the gate/up kernel has no
// registers for it.
#ifndef Q3_GEMM_CVT_LDS
#define Q3_GEMM_CVT_LDS 3
#endif
// 1: for fp32 outputs (with residual), the direct-to-LDS kernel computes C^T blocks (weight
// fragment as the MFMA A operand), so each lane ends up with runs of 4 consecutive output
// columns of one row: one 16-byte residual load and store per run instead of four 4-byte ones.
// (For 16-bit outputs the untransposed layout, 64 contiguous bytes per row and store, measured
// faster.)
// 1: direct-to-LDS loads through buffer descriptors where the operands fit 32-bit offsets
#ifndef Q3_GEMM_BUF
#define Q3_GEMM_BUF 1
#endif
#ifndef Q3_GEMM_TRANS
#define Q3_GEMM_TRANS 1
#endif
// 1: fp32 outputs of the 256 x 256 tile leave through LDS as whole 256-byte row segments
// 1: the gate/up SwiGLU GEMM runs as persistent workgroups (one per CU, several tiles each)
#ifndef Q3_GEMM_PERSIST
#define Q3_GEMM_PERSIST 1
#endif
#ifndef Q3_GEMM_LDS_EPI
#define Q3_GEMM_LDS_EPI 1
#endif
// 1: each K step's fragment reads and MFMAs in fixed scheduling groups (see the step)
#ifndef Q3_GEMM_SGG
#define Q3_GEMM_SGG 1
#endif
// 1: one-tile fp32-residual products take the residual in chunks during their first K steps
#ifndef Q3_GEMM_RSTREAM
#define Q3_GEMM_RSTREAM 1
#endif

namespace q3 {

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order
template <int N, int I = 0, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

constexpr int kBM = 256;
constexpr int kBK = 64;  // K must be a multiple of this

// Workgroup id -> (tile row, tile column). Hardware dispatches ids round-robin over the 8
// XCDs; ids are first regrouped so that XCD x gets a contiguous range of logical ids, then
// logical ids walk GM tile-rows at a time so concurrently running tiles share operands.
__device__ __forceinline__ void tile_coords(int bid, int nwg, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  int L = bid;
  if ((nwg & 7) == 0) L = (bid & 7) * (nwg >> 3) + (bid >> 3);
  constexpr int GM = 4;  // 4 measured best on the 8B shapes (o-proj 3-5% faster than 8 or 16)
  const int per_group = GM * tiles_n;
  const int group = L / per_group;
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_group = L - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// Source row of B for LDS tile row r of tile column tn.
template <int BN, int WN, int EPI>
__device__ __forceinline__ const uint16_t* b_row(const GemmParams& p, int tn, int r) {
  if (EPI == EPI_SWIGLU_16) {
    // Tile tn covers F columns [tn*BN/2, tn*BN/2 + BN/2). LDS rows come in segments of half a
    // wave's column width, alternating gate and up, so that each wave's columns hold gate
    // columns followed by the up columns of the same F range: the SwiGLU pairing is then
    // lane-local in the accumulators.
    constexpr int SEG = BN / WN / 2;
    const int seg = r / SEG;
    const int f = tn * (BN / 2) + (seg >> 1) * SEG + (r % SEG);
    return ((seg & 1) ? p.B1 : p.B0) + static_cast<int64_t>(f) * p.ldb;
  } else {
    const int n = tn * BN + r;
    if (n < p.nseg0) return p.B0 + static_cast<int64_t>(n) * p.ldb;
    if (n < p.nseg1) return p.B1 + static_cast<int64_t>(n - p.nseg0) * p.ldb;
    return p.B2 + static_cast<int64_t>(n - p.nseg1) * p.ldb;
  }
}

// Segment of B holding LDS tile row r of tile column tn (the same rows b_row reads): base
// pointer, row index within the segment, and the segment's row count.
template <int BN, int WN, int EPI>
__device__ __forceinline__ void b_seg(const GemmParams& p, int tn, int r, const uint16_t*& base,
                                      int& idx, int& rows) {
  if (EPI == EPI_SWIGLU_16) {
    constexpr int SEG = BN / WN / 2;
    const int seg = r / SEG;
    base = (seg & 1) ? p.B1 : p.B0;
    idx = tn * (BN / 2) + (seg >> 1) * SEG + (r % SEG);
    rows = p.N / 2;
  } else {
    const int n = tn * BN + r;
    if (n < p.nseg0) {
      base = p.B0; idx = n; rows = p.nseg0;
    } else if (n < p.nseg1) {
      base = p.B1; idx = n - p.nseg0; rows = p.nseg1 - p.nseg0;
    } else {
      base = p.B2; idx = n - p.nseg1; rows = p.N - p.nseg1;
    }
  }
}

// silu(g) = g / (1 + e^-g), the quotient through the hardware reciprocal (about 1 ulp of fp32,
// far below the 16-bit rounding of the stored product)
__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Epilogue shared by the kernels: stores a wave's accumulators. Accumulator element e of
// block (mi, ni) in lane l holds row 8*(e/4) + 4*(l/32) + e%4 and column l%32 of that block.
template <int BN, int WM, int WN, int EPI, int OP, bool TRANS = false, bool RIN = false, bool CT = false>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& p,
                                              f32x16 (&acc)[kBM / WM / 32][BN / WN / 32], int tm,
                                              int tn, int wm, int wn, int lane) {
  using F = Fmt<OP>;
  constexpr int MI = kBM / WM / 32;
  constexpr int NI = BN / WN / 32;
  // SwiGLU output element (m, f): row-major m * ldc + f, or (CT) tiled with ldc == F
  auto c_row = [&](int m) -> int64_t {
    return CT ? static_cast<int64_t>(m >> 4) * 16 * p.ldc + (m & 15) * 32 : static_cast<int64_t>(m) * p.ldc;
  };
  auto c_col = [&](int f) { return CT ? (f >> 5) * 512 + (f & 31) : f; };
  if (TRANS) {
    // acc[mi][ni] holds the transposed block: lane l has row m = l%32 of block mi and, in
    // elements 4q..4q+3, the four consecutive columns 8q + 4*(l/32) + 0..3 of block ni
    const int m = tm * kBM + wm * (32 * MI) + (lane & 31);
    const int c4 = 4 * (lane >> 5);
    if (m >= p.M) return;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = m + mi * 32;
      if (row >= p.M) break;
      if (EPI == EPI_SWIGLU_16) {
        uint16_t* C = static_cast<uint16_t*>(p.C) + c_row(row);
#pragma unroll
        for (int ni = 0; ni < NI / 2; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int f = tn * (BN / 2) + wn * (16 * NI) + ni * 32 + 8 * q + c4;
            float h[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              h[r] = silu_f(acc[mi][ni][4 * q + r]) * (acc[mi][ni + NI / 2][4 * q + r] * p.act_scale);
            *reinterpret_cast<u32x2*>(C + c_col(f)) = u32x2{F::pack2(h[0], h[1]), F::pack2(h[2], h[3])};
          }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = tn * BN + wn * 32 * NI + ni * 32 + 8 * q + c4;
            const f32x16& a = acc[mi][ni];
            const float sc = p.out_scale;
            if (EPI == EPI_STORE_16) {
              uint16_t* C = static_cast<uint16_t*>(p.C) + static_cast<int64_t>(row) * p.ldc + n;
              *reinterpret_cast<u32x2*>(C) = u32x2{F::pack2(a[4 * q] * sc, a[4 * q + 1] * sc),
                                                   F::pack2(a[4 * q + 2] * sc, a[4 * q + 3] * sc)};
            } else {
              // with RIN the accumulators started from R / out_scale
              f32x4 v = {a[4 * q] * sc, a[4 * q + 1] * sc, a[4 * q + 2] * sc, a[4 * q + 3] * sc};
              if (!RIN && p.R) {
                const f32x4 r = *reinterpret_cast<const f32x4*>(p.R + static_cast<int64_t>(row) * p.ldr + n);
                v += r;
              }
              *reinterpret_cast<f32x4*>(static_cast<float*>(p.C) + static_cast<int64_t>(row) * p.ldc + n) = v;
            }
          }
      }
    }
    return;
  }
  const int col_in_blk = lane & 31;
  const int row_base = tm * kBM + wm * (32 * MI) + 4 * (lane >> 5);
  if (EPI == EPI_SWIGLU_16) {
    // Row row_base + mi*32 + 8*(e/4) + e%4 (row_base % 16 is 0 or 4, so no offset below
    // carries into the next 16-row group) and column f0 + ni*32 (f0 % 32 = the lane's column):
    // the element offset is a per-lane base plus a constant multiple of ldc plus a constant.
    static_assert((32 * MI) % 16 == 0, "row groups");
    const int f0 = tn * (BN / 2) + wn * (16 * NI) + col_in_blk;
    uint16_t* C = static_cast<uint16_t*>(p.C) + c_row(row_base) + c_col(f0);
    auto off = [&](int mi, int ni, int e) -> int64_t {
      if (CT)
        return static_cast<int64_t>(2 * mi + (e >> 3)) * 16 * p.ldc + (8 * ((e >> 2) & 1) + (e & 3)) * 32 + ni * 512;
      return static_cast<int64_t>(mi * 32 + 8 * (e >> 2) + (e & 3)) * p.ldc + ni * 32;
    };
    // tiles wholly inside M (all but a ragged last row of tiles) store without per-row checks
    auto store_all = [&](auto check) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI / 2; ++ni) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = row_base + mi * 32 + 8 * (e >> 2) + (e & 3);
            if (!check.value || m < p.M) {
              const float g = acc[mi][ni][e];
              const float u = acc[mi][ni + NI / 2][e];
              C[off(mi, ni, e)] = F::from_f32(silu_f(g) * (u * p.act_scale));
            }
          }
        }
    };
    if (tm * kBM + kBM <= p.M) store_all(std::false_type{});
    else store_all(std::true_type{});
  } else {
    // as above: a per-lane base (row row_base, column n0) plus constant multiples of ldc
    const int n0 = tn * BN + wn * 32 * NI + col_in_blk;
    uint16_t* C16 = static_cast<uint16_t*>(p.C) + static_cast<int64_t>(row_base) * p.ldc + n0;
    auto store_all = [&](auto check) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int n = n0 + ni * 32;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = row_base + mi * 32 + 8 * (e >> 2) + (e & 3);
            if (!check.value || m < p.M) {
              const float v = acc[mi][ni][e] * p.out_scale;
              if (EPI == EPI_STORE_16) {
                C16[static_cast<int64_t>(mi * 32 + 8 * (e >> 2) + (e & 3)) * p.ldc + ni * 32] = F::from_f32(v);
              } else {
                float r = 0.f;
                if (p.R) r = p.R[static_cast<int64_t>(m) * p.ldr + n];
                static_cast<float*>(p.C)[static_cast<int64_t>(m) * p.ldc + n] = r + v;
              }
            }
          }
        }
    };
    if (tm * kBM + kBM <= p.M) store_all(std::false_type{});
    else store_all(std::true_type{});
  }
}

// ---------------------------------------------------------------------------------------
// Direct-to-LDS variant: tiles go from global memory straight into LDS with
// global_load_lds_dwordx4 (lane i of a wave instruction fills the i-th 16-byte slot of a
// contiguous 1 KiB block), through a 4-stage ring of 32-wide K steps, so each tile is requested
// three K steps before its MFMAs and no registers hold staged data. A row of a stage is 64 bytes
// (4 chunks); the chunk a slot holds is XOR-permuted by row so that the 32-row fragment reads hit
// distinct banks. bf16 weights feeding fp16 products are converted after the fragment read.
constexpr int kBK2 = 32;

__device__ __forceinline__ int swz4(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
// Tiled operands: a load instruction's 64 lanes fill the 64 slots of 16 LDS rows from one 1 KiB
// tile; lane l takes the tile's chunk (row l/4, chunk (l%4) ^ swz4(l/4)), so the LDS holds the
// same permuted rows as for row-major operands (swz4 depends on the row's low 4 bits only).
__device__ __forceinline__ int tile_pos(int lane) { return (lane & ~3) | ((lane & 3) ^ swz4(lane >> 2)); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void g2lds(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}
// The same 16-byte direct-to-LDS load through a buffer descriptor: byte offset voff (per lane)
// plus soff (scalar).
__device__ __forceinline__ void buf2lds(__amdgpu_buffer_rsrc_t r, void* l, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 16, voff, soff, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define Q3_WAIT_VMCNT(N) \
  __builtin_amdgcn_s_waitcnt(((N) & 0xF) | (0x7 << 4) | (0xF << 8) | (((N) >> 4) << 14))

// Q4_0 weight tiles (GGML's block: a binary16 scale d, then 16 bytes holding the codes of
// weights j (low nibble) and j + 16 (high nibble) of 32 consecutive weights of a row; weight =
// d * (code - 8)). One 32-wide K step of a weight row is exactly one 18-byte block, and two
// consecutive blocks (36 bytes) start at a 4-byte boundary when K is a multiple of 64. One
// thread per weight row loads the pair on even K steps and decodes block 0 of it on the even
// step, block 1 on the odd one. Each weight is d * (code - 8) rounded once to the operand type,
// as the separate expansion kernel does: the code becomes the binary16 1024 + code by inserting
// its byte under a 0x64 exponent byte, 1032 is subtracted exactly, and one multiplication by d
// rounds.
typedef uint32_t u32x4a4_g __attribute__((ext_vector_type(4), aligned(4)));
struct Q4Pair {
  u32x4 a, b;   // bytes 0-15, 16-31 of the pair
  uint32_t c;   // bytes 32-35
};
// The 4 chunks of 8 weights (chunk i: weights 8i .. 8i+7) of block `second` of the pair.
template <int OP>
__device__ __forceinline__ void q4_decode_block(const Q4Pair& q, bool second, u32x4 (&chunk)[4]) {
  // block 0: d in bytes 0-1, codes in bytes 2-17; block 1: d in bytes 18-19, codes 20-35
  const uint32_t w[9] = {q.a[0], q.a[1], q.a[2], q.a[3], q.b[0], q.b[1], q.b[2], q.b[3], q.c};
  uint32_t code[4];
  uint32_t dbits;
  if (second) {
    dbits = w[4] >> 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) code[i] = w[5 + i];
  } else {
    dbits = w[0] & 0xFFFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) code[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], 2u);
  }
  // code[i] holds code bytes 4i .. 4i+3: low nibbles = weights 4i..4i+3 (chunk i / 2), high
  // nibbles = weights 16 + 4i .. (chunk 2 + i / 2)
  if constexpr (OP == OP_F16) {
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    const h2_t dd = __builtin_bit_cast(h2_t, dbits | (dbits << 16));
    const h2_t off = __builtin_bit_cast(h2_t, 0xE408E408u);  // (-1032, -1032)
    auto pair = [&](uint32_t nib, uint32_t sel) {
      const h2_t v = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, nib, sel)) + off;
      return __builtin_bit_cast(uint32_t, v * dd);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = code[i] & 0x0F0F0F0Fu, hi = (code[i] >> 4) & 0x0F0F0F0Fu;
      chunk[i >> 1][2 * (i & 1)] = pair(lo, 0x04010400u);
      chunk[i >> 1][2 * (i & 1) + 1] = pair(lo, 0x04030402u);
      chunk[2 + (i >> 1)][2 * (i & 1)] = pair(hi, 0x04010400u);
      chunk[2 + (i >> 1)][2 * (i & 1) + 1] = pair(hi, 0x04030402u);
    }
  } else {
    const float d = h2f(static_cast<uint16_t>(dbits));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t b0 = (code[i] >> (16 * k)) & 0xFFu, b1 = (code[i] >> (16 * k + 8)) & 0xFFu;
        chunk[i >> 1][2 * (i & 1) + k] = pack2bf(d * static_cast<float>(static_cast<int>(b0 & 15u) - 8),
                                                 d * static_cast<float>(static_cast<int>(b1 & 15u) - 8));
        chunk[2 + (i >> 1)][2 * (i & 1) + k] = pack2bf(d * static_cast<float>(static_cast<int>(b0 >> 4) - 8),
                                                       d * static_cast<float>(static_cast<int>(b1 >> 4) - 8));
      }
  }
}

// TA: A in the tiled layout (and, for EPI_SWIGLU_16, the output too); TB: B tiled.
template <int BN, int WM, int WN, int EPI, int OP, bool CVT, int NS, bool BUF, bool BQ = false, bool TA = false,
          bool TB = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WM * WN, 64 * WM * WN),
                          amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4)))
void gemm_d2l_kernel(const GemmParams p) {
  using F = Fmt<OP>;
  constexpr int THREADS = 64 * WM * WN;
  constexpr int MI = kBM / WM / 32;
  constexpr int NI = BN / WN / 32;
  constexpr int ASLOT = kBM * 4;              // 16-byte slots per stage, A
  constexpr int BSLOT = BN * 4;               // 16-byte slots per stage, B
  constexpr int WAVES = THREADS / 64;
  constexpr int AJ = ASLOT / THREADS;         // loads per thread per stage, A
  constexpr int BJ = (BSLOT + THREADS - 1) / THREADS;  // loads per thread per stage, B
  constexpr int LPS = AJ + (BQ ? 0 : BJ);     // loads per thread per stage (equal in every wave)
  // BQ: Q4_0 block pairs are requested with the stages of even K steps, 3 loads each
  constexpr int QL = 3;
  static_assert(!BQ || (!CVT && NS % 2 == 0 && BN <= THREADS), "Q4_0 weight tiles");
  // loads this thread issues for stage st (the K step of stage st has the parity of st)
  auto lps = [](int st) constexpr { return LPS + ((BQ && st % 2 == 0) ? QL : 0); };
  constexpr bool SINK = (BSLOT % THREADS) != 0;
  constexpr bool TRANS = Q3_GEMM_TRANS && EPI == EPI_STORE_F32;  // accumulators hold C^T blocks
  static_assert(ASLOT % THREADS == 0 && BSLOT % 64 == 0, "tile shape");
  static_assert(NS >= 4 && NS * (ASLOT + BSLOT) * 16 + (SINK ? 1024 : 0) <= 160 * 1024, "LDS");
  // NS stages of the A and B tiles; with SINK, the waves past the last B block repeat a valid
  // load into one extra block that is never read, so every wave issues LPS loads per stage
  // and one s_waitcnt immediate fits all of them.
  // One array per stage (not one 2-D array): the compiler can then tell the stage a DMA
  // writes from the stages being read, and adds no wait of its own before the reads.
  constexpr int BSZ = BSLOT + (SINK ? 64 : 0);
  __shared__ u32x4 sA0[ASLOT], sA1[ASLOT], sA2[ASLOT], sA3[ASLOT], sA4[NS > 4 ? ASLOT : 1];
  __shared__ u32x4 sB0[BSZ], sB1[BSZ], sB2[BSZ], sB3[BSZ], sB4[NS > 4 ? BSZ : 1];
  auto stA = [&](int st) -> u32x4* {
    return st == 0 ? sA0 : st == 1 ? sA1 : st == 2 ? sA2 : st == 3 ? sA3 : sA4;
  };
  auto stB = [&](int st) -> u32x4* {
    return st == 0 ? sB0 : st == 1 ? sB1 : st == 2 ? sB2 : st == 3 ? sB3 : sB4;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int tiles_m = (p.M + kBM - 1) / kBM;
  const int tiles_n = p.N / BN;
  const int ntiles = tiles_m * tiles_n;
  // Persistent form (SwiGLU output): a grid smaller than the tile count walks tiles
  // blockIdx.x, + gridDim.x, ... (each the tile a one-tile-per-workgroup launch would give that
  // workgroup id, on the same XCD when gridDim.x % 8 == 0); the LDS ring runs on across tile
  // boundaries, so the next tile's first K steps load during this tile's last ones and its
  // epilogue. The host launches it only when 4 divides the K steps of a tile.
  const int my_tiles = (ntiles - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                       static_cast<int>(gridDim.x);
  int tm, tn;  // the tile being computed
  tile_coords(blockIdx.x, ntiles, tiles_m, tiles_n, tm, tn);

  // Load slot of this lane in pass j: the wave's 64 consecutive slots starting at
  // (wave + j*waves)*64; slot -> tile row slot/4, stored chunk slot%4, global chunk
  // (slot%4) ^ swz4(row). The per-tile part (rows of A, rows of B) is set by set_issue_tile
  // for the tile whose K steps are being requested.
  const uint16_t* a_src[AJ];
  const uint16_t* b_src[BJ];
  // BUF: the same loads through buffer descriptors. A load instruction covers 16 tile rows
  // (one B segment: the host checks segment bounds are multiples of 16), so its descriptor is
  // uniform; per-lane byte offsets are fixed for a tile and the K step goes into the scalar
  // offset, which leaves no address arithmetic in the loop.
  __amdgpu_buffer_rsrc_t rsrc_a, rsrc_b[BJ];
  uint32_t voff_a[AJ], voff_b[BJ];
  if constexpr (BUF)
    rsrc_a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.A), static_cast<short>(0),
                                               static_cast<int>(2 * static_cast<int64_t>(TA ? (p.M + 15) & ~15 : p.M) * p.lda),
                                               0x00020000);
  // per K step, the operands advance 32 elements (row-major) or one 512-element tile (tiled);
  // as shifts of k0 (elements) to element and byte offsets
  constexpr int a_ksh = TA ? 4 : 0, b_ksh = TB ? 4 : 0;
  // BQ: this thread's weight row (one thread per row; threads past BN load row BN - 1 and store
  // nothing)
  const int q_r = min(tid, BN - 1);
  const bool q_active = tid < BN;
  const int64_t q_row_bytes = static_cast<int64_t>(p.K / 32) * 18;
  const uint8_t* q_rowp = nullptr;
  auto set_issue_tile = [&](int itm, int itn) {
    if constexpr (BQ) {
      const uint16_t* base;
      int idx, rows;
      b_seg<BN, WN, EPI>(p, itn, q_r, base, idx, rows);
      q_rowp = reinterpret_cast<const uint8_t*>(base) + idx * q_row_bytes;
    }
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
      const int slot = (wave + j * WAVES) * 64 + lane;
      const int row = slot >> 2;
      if constexpr (TA) {
        // the load's 16 rows are one row group (groups past the last one read the last)
        const int g = min(itm * (kBM / 16) + (slot >> 6), (p.M + 15) / 16 - 1);
        a_src[j] = p.A + static_cast<int64_t>(g) * 16 * p.K + tile_pos(lane) * 8;
      } else {
        const int r = min(itm * kBM + row, p.M - 1);  // rows past M are read, never stored
        a_src[j] = p.A + static_cast<int64_t>(r) * p.lda + ((slot & 3) ^ swz4(row)) * 8;
      }
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      const int blk = wave + j * WAVES;
      int slot = blk * 64 + lane;
      if (slot >= BSLOT) slot = lane;  // sink load: a valid row
      const int row = slot >> 2;
      // first tile row of this load's 16, from wave-uniform values only: the segment base
      // then is provably uniform and its buffer descriptor needs no per-lane loop
      const int row0 = blk * 64 < BSLOT ? blk * 16 : 0;
      const uint16_t* base;
      int idx0, rows;
      b_seg<BN, WN, EPI>(p, itn, row0, base, idx0, rows);
      // tiled B: a load's 16 rows are one row group of one segment (the host checks that
      // segment bounds are multiples of 16)
      b_src[j] = TB ? base + static_cast<int64_t>(idx0 >> 4) * 16 * p.K + tile_pos(lane) * 8
                           : b_row<BN, WN, EPI>(p, itn, row) + ((slot & 3) ^ swz4(row)) * 8;
      if constexpr (BUF)
        rsrc_b[j] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), static_cast<short>(0),
                                                      static_cast<int>(2 * static_cast<int64_t>(rows) * p.ldb), 0x00020000);
      if constexpr (BUF) voff_b[j] = static_cast<uint32_t>(2 * (b_src[j] - base));
    }
    if constexpr (BUF) {
#pragma unroll
      for (int j = 0; j < AJ; ++j)
        voff_a[j] = static_cast<uint32_t>(2 * (a_src[j] - p.A));
    }
  };
  set_issue_tile(tm, tn);

  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
  // fp32 output with a residual: the accumulators start from R (C^T layout: lane l, elements
  // 4q..4q+3 of block (mi, ni) = R[row l%32 of block mi][4 columns 8q + 4*(l/32) ..]), loaded
  // here, behind the ring's first tile loads, so the epilogue only stores; rows past M load a
  // clamped valid row and are never stored
  const bool rin = TRANS && p.R != nullptr;
  // the residual enters the accumulators divided by out_scale (exact for a power of two), so
  // the epilogue's single multiplication by out_scale leaves it unchanged
  const float r_scale = 1.0f / p.out_scale;
  // RS: a one-tile workgroup with enough K steps takes the residual in MI * NI chunks (one
  // 32 x 32 accumulator block each) during its first groups of K steps instead of before them,
  // so a launch's residual reads (all workgroups at once) spread over the K loop instead of
  // stalling the first MFMA; the sum is the same up to the order of fp32 additions
  // (instantiated for the layer's products only: buffer loads, tiled activations)
  constexpr bool RS_OK = Q3_GEMM_RSTREAM && TRANS && EPI == EPI_STORE_F32 && BUF && TA;
  constexpr int RS_GAP = 2;  // groups of NS steps from one chunk to the next
  const bool rs = RS_OK && rin && my_tiles == 1 && p.K / kBK2 >= NS * RS_GAP * MI * NI;
  // C^T layout of the residual: lane l, elements 4q..4q+3 of block (mi, ni) = R[row l%32 of
  // block mi][4 columns 8q + 4*(l/32) ..]; rows past M read a clamped valid row (never stored)
  auto r_load = [&](int mi, int ni, f32x16& dst) __attribute__((always_inline)) {
    const int c4 = 4 * (lane >> 5);
    const int row = min(tm * kBM + wm * (32 * MI) + mi * 32 + (lane & 31), p.M - 1);
    const float* rr = p.R + static_cast<int64_t>(row) * p.ldr;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 r = *reinterpret_cast<const f32x4*>(rr + tn * BN + wn * 32 * NI + ni * 32 + 8 * q + c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[4 * q + e] = r[e] * r_scale;
    }
  };
  if (rin && !rs) {
    const int c4 = 4 * (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = min(tm * kBM + wm * (32 * MI) + mi * 32 + (lane & 31), p.M - 1);
      const float* rr = p.R + static_cast<int64_t>(row) * p.ldr;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 r = *reinterpret_cast<const f32x4*>(rr + tn * BN + wn * 32 * NI + ni * 32 + 8 * q + c4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mi][ni][4 * q + e] = r[e] * r_scale;
        }
    }
  }

  // STAGE_B: B tiles come through registers (one 16-byte load per slot), are converted once
  // and stored to LDS by the same thread before the barrier that publishes the stage
  constexpr bool STAGE_B = CVT && Q3_GEMM_CVT_LDS == 3 && WM >= 4;
  u32x4 breg[NS][BJ];
  Q4Pair qraw[NS / 2];   // BQ: the block pair of stages 2i (block 0) and 2i + 1 (block 1)
  const int nk = p.K / kBK2;
  const int total = my_tiles * nk;  // K steps of all this workgroup's tiles, in order
  // Requests go out one K step at a time in order: (iss_tile, iss_kt) is the next one; past
  // the last step the last one is requested again (never used).
  int iss_tile = 0, iss_kt = 0;
  auto issue = [&](int st, int g) {
    int k0;
    if (g < total) {
      if (iss_kt == nk) {
        iss_kt = 0;
        ++iss_tile;
        int itm, itn;
        tile_coords(blockIdx.x + iss_tile * gridDim.x, ntiles, tiles_m, tiles_n, itm, itn);
        set_issue_tile(itm, itn);
      }
      k0 = iss_kt * kBK2;
      ++iss_kt;
    } else {
      k0 = (nk - 1) * kBK2;
    }
    if constexpr (BQ) {
      if (st % 2 == 0) {   // even K step: its block and the next one, 36 bytes from a 4-byte boundary
        const uint8_t* src = q_rowp + (k0 / 64) * 36;
        const u32x4a4_g v0 = *reinterpret_cast<const u32x4a4_g*>(src);
        const u32x4a4_g v1 = *reinterpret_cast<const u32x4a4_g*>(src + 16);
        Q4Pair& q = qraw[st / 2];
        q.a = u32x4{v0[0], v0[1], v0[2], v0[3]};
        q.b = u32x4{v1[0], v1[1], v1[2], v1[3]};
        q.c = *reinterpret_cast<const uint32_t*>(src + 32);
      }
    }
    const int ka = k0 << a_ksh, kb = k0 << b_ksh;  // element offsets of this K step
    if constexpr (BUF) {
#pragma unroll
      for (int j = 0; j < AJ; ++j)
        buf2lds(rsrc_a, stA(st) + (wave + j * WAVES) * 64, voff_a[j], 2 * ka);
      if constexpr (!BQ)
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        const int blk = wave + j * WAVES;
        if constexpr (STAGE_B)
          breg[st][j] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_b[j], voff_b[j], 2 * kb, 0);
        else
          buf2lds(rsrc_b[j], stB(st) + (blk * 64 < BSLOT ? blk : BSLOT / 64) * 64, voff_b[j], 2 * kb);
      }
    } else {
#pragma unroll
      for (int j = 0; j < AJ; ++j) g2lds(a_src[j] + ka, stA(st) + (wave + j * WAVES) * 64);
      if constexpr (!BQ)
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        const int blk = wave + j * WAVES;
        if constexpr (STAGE_B)
          breg[st][j] = *reinterpret_cast<const u32x4*>(b_src[j] + kb);
        else
          g2lds(b_src[j] + kb, stB(st) + (blk * 64 < BSLOT ? blk : BSLOT / 64) * 64);
      }
    }
  };
  const int fr = lane & 31;
  const int fh = lane >> 5;
  // Fragment sets: set 0 holds sub-step 0 of a K step, set 1 sub-step 1.
  u32x4 fa[2][MI], fb[2][NI];
  auto fread = [&](int st, int ks, int set) {
    const int ch = ks * 2 + fh;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * (32 * MI) + mi * 32 + fr;
      fa[set][mi] = stA(st)[row * 4 + (ch ^ swz4(row))];
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int row = wn * (32 * NI) + ni * 32 + fr;
      fb[set][ni] = stB(st)[row * 4 + (ch ^ swz4(row))];
    }
  };
  // Where the bf16 -> fp16 weight conversion happens (Q3_GEMM_CVT_LDS): per fragment after the
  // read, in LDS once per workgroup, or (STAGE_B) once per workgroup on the way into LDS.
  constexpr bool CVT_IN_LDS = CVT && (Q3_GEMM_CVT_LDS == 1 ? WM >= 4 : Q3_GEMM_CVT_LDS == 2);
  constexpr bool CVT_FRAG = CVT && !CVT_IN_LDS && !STAGE_B;
  auto mfmas = [&](int set) {
    u32x4 bv[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      bv[ni] = fb[set][ni];
      if (CVT_FRAG) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[ni][e] = bf16x2_to_f16x2(bv[ni][e]);
      }
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = TRANS ? F::mfma(bv[ni], fa[set][mi], acc[mi][ni])
                            : F::mfma(fa[set][mi], bv[ni], acc[mi][ni]);
  };
  // In-LDS conversion of the B slots this thread loaded into stage st (its own loads of that
  // stage must have landed).
  auto convert_own = [&](int st) {
    if constexpr (BQ) {
      // the K step held by stage st has the parity of st (NS and the K steps per tile are even)
      if (q_active) {
        u32x4 chunk[4];
        q4_decode_block<OP>(qraw[st / 2], (st & 1) != 0, chunk);
#pragma unroll
        for (int c = 0; c < 4; ++c) stB(st)[q_r * 4 + (c ^ swz4(q_r))] = chunk[c];
      }
    }
    if constexpr (STAGE_B) {
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        const int blk = wave + j * WAVES;
        if (blk * 64 < BSLOT) {
          u32x4 v = breg[st][j];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = bf16x2_to_f16x2(v[e]);
          stB(st)[blk * 64 + lane] = v;
        }
      }
    }
    if (CVT_IN_LDS) {
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        const int blk = wave + j * WAVES;
        if (blk * 64 < BSLOT) {
          u32x4 v = stB(st)[blk * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = bf16x2_to_f16x2(v[e]);
          stB(st)[blk * 64 + lane] = v;
        }
      }
    }
  };
  // s_waitcnt vmcnt(N) (others unconstrained) / lgkmcnt(0) + workgroup barrier; the empty asm
  // statements keep the compiler from moving memory accesses across them.
  auto wait_vm = [&](auto n_vm) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((decltype(n_vm)::value & 0xF) | (0x7 << 4) | (0xF << 8) |
                               ((decltype(n_vm)::value >> 4) << 14));
    asm volatile("" ::: "memory");
  };
  // Workgroup barrier. With wait_lds, this thread's LDS accesses complete first (lgkmcnt(0)):
  // needed where threads write LDS before it (converted or decoded weight tiles, the LDS
  // epilogue). In a ring filled only by direct-to-LDS loads (covered by the vmcnt waits), the
  // newest MI + NI LDS reads may stay in flight across a step barrier: they are the next
  // stage's first sub-step fragments, and the loads issued after the barrier refill the stage
  // before that one. Every older read must be done, though: the compiler moves a step's last
  // MFMAs, and the waits for their fragments with them, past the next barrier, and a read of the
  // stage being refilled still in flight there would race with its direct-to-LDS write. LDS
  // reads complete in order; scalar loads counted by the same counter only make the wait
  // stricter.
  auto barrier = [&](auto wait_lds) {
    asm volatile("" ::: "memory");
    if constexpr (decltype(wait_lds)::value)
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (0x3 << 14));  // lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (0x3 << 14) | ((MI + NI) << 8));  // lgkmcnt(MI + NI)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  constexpr bool LDS_W = STAGE_B || CVT_IN_LDS || BQ;  // threads write ring stages themselves
  static_assert(MI + NI <= 15, "lgkmcnt immediate");
  using WaitLds = std::integral_constant<bool, LDS_W>;

#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st, st);
  // own loads of stage 0 landed (those of stages 1 .. NS-2 may still be in flight)
  constexpr int W0 = [&]() constexpr {
    int n = 0;
    for (int st = 1; st < NS - 1; ++st) n += lps(st);
    return n;
  }();
  wait_vm(std::integral_constant<int, W0>{});
  convert_own(0);
  barrier(WaitLds{});  // stage 0 complete (and converted) everywhere
  fread(0, 0, 0);
  // Step kt (stage kt % NS): wait for this thread's loads of stage kt+1 (later stages may still
  // be in flight) and convert them, barrier (stage kt+1 complete everywhere; every wave is past
  // its reads of stage kt-1), refill stage kt-1's buffer with step kt+NS-1, then the two
  // 16-wide sub-steps; the second one reads sub-step 0 of step kt+1, so the MFMAs after the
  // next barrier start on operands already in registers.
  // RS chunk in flight: loaded at step u = 0 of a group (after its tile requests), 4 loads per
  // lane; steps 1 and 2 of the group let them stay outstanding, step 3 waits for them (they
  // are older than the stage it waits for) and adds them
  f32x16 rtmp;
  constexpr int RL = 4;
  static_assert(NS == 4, "residual streaming assumes a 4-stage ring");
  auto step = [&](auto u_c, int g, auto rc_c) __attribute__((always_inline)) {
    constexpr int u = decltype(u_c)::value;
    constexpr int rc = decltype(rc_c)::value;  // residual block mi * NI + ni of this group, or -1
    // own loads of stage u+1 landed (stages u+2 .. u+NS-2 may still be in flight)
    constexpr int WN1 = [&]() constexpr {
      int n = 0;
      for (int k = 2; k <= NS - 2; ++k) n += lps((u + k) % NS);
      return n;
    }() + ((rc >= 0 && (u == 1 || u == 2)) ? RL : 0);
    wait_vm(std::integral_constant<int, WN1>{});
    if constexpr (rc >= 0 && u == NS - 1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rc / NI][rc % NI][e] += rtmp[e];
    }
    convert_own((u + 1) % NS);
    barrier(WaitLds{});
    issue((u + NS - 1) % NS, g + NS - 1);
    if constexpr (rc >= 0 && u == 0) r_load(rc / NI, rc % NI, rtmp);
    fread(u, 1, 1);
    mfmas(0);
    fread((u + 1) % NS, 0, 0);
    mfmas(1);
#if Q3_GEMM_SGG
    // scheduling groups in source order: each sub-step's fragment reads are issued before the
    // MFMAs of the other sub-step (the compiler otherwise moved them among those MFMAs, so the
    // MFMAs right after them waited for LDS): QKV, o-proj and down ~2% faster
    __builtin_amdgcn_sched_group_barrier(0x100, MI + NI, 0);   // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);   // MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, MI + NI, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);
#endif
  };
  using NoR = std::integral_constant<int, -1>;
  // Whole groups of NS steps without any branch (stage indices are constants after unrolling),
  // then the remaining steps (one-tile launches whose K steps are not a multiple of NS). With
  // several tiles per workgroup (NS divides a tile's K steps, so every tile ends with a group),
  // a finished tile's epilogue runs right after its last group: the next tile's first sub-step
  // fragments are already in registers and its first stages are on their way.
  int g = 0;
  int done = 0, cur = 0;
  if constexpr (RS_OK) {
    if (rs) {
      // chunk c in group c * RS_GAP, plain groups in between
      static_for<MI * NI>([&](auto c_c) __attribute__((always_inline)) {
        static_for<NS>([&](auto u_c) __attribute__((always_inline)) { step(u_c, g + decltype(u_c)::value, c_c); });
        g += NS;
        for (int k = 1; k < RS_GAP; ++k, g += NS)
          static_for<NS>([&](auto u_c) __attribute__((always_inline)) { step(u_c, g + decltype(u_c)::value, NoR{}); });
      });
    }
  }
  for (; g + NS <= total; g += NS) {
    static_for<NS>([&](auto u_c) __attribute__((always_inline)) { step(u_c, g + decltype(u_c)::value, NoR{}); });
    if constexpr (EPI == EPI_SWIGLU_16) {
      const bool tile_end = my_tiles > 1 && done + NS == nk;
      if (my_tiles > 1) done += NS;
      if (tile_end) {
        done = 0;
        gemm_epilogue<BN, WM, WN, EPI, OP, TRANS, false, TA>(p, acc, tm, tn, wm, wn, lane);
        if (g + NS < total) {
          ++cur;
          tile_coords(blockIdx.x + cur * gridDim.x, ntiles, tiles_m, tiles_n, tm, tn);
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;
        }
      }
    }
  }
  static_for<NS - 1>([&](auto u_c) __attribute__((always_inline)) {
    if (g + decltype(u_c)::value < total) step(u_c, g + decltype(u_c)::value, NoR{});
  });

  // the trailing reloads of the last tile must land before this workgroup's LDS is released
  Q3_WAIT_VMCNT(0);
  if (my_tiles > 1) return;  // every tile's epilogue already ran
  constexpr bool LDS_EPI = Q3_GEMM_LDS_EPI && TRANS && EPI == EPI_STORE_F32 && WM == 2 && WN == 4 && BN == 256;
  if constexpr (LDS_EPI) {
    // fp32 output (residual already in the accumulators) through LDS: each wave owns one 16 KiB
    // ring array and stages half of its 128 x 64 block at a time (chunk of 4 columns XOR-permuted
    // by row), then writes whole 256-byte row segments (16 lanes per row)
    barrier(std::true_type{});  // every wave is past its last fragment reads of the ring
    u32x4* buf = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sA2 : wave == 3 ? sA3
               : wave == 4 ? sB0 : wave == 5 ? sB1 : wave == 6 ? sB2 : sB3;
    float* C = static_cast<float*>(p.C);
#pragma unroll
    for (int half = 0; half < MI / 2; ++half) {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const int r = m2 * 32 + fr;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ch = ni * 8 + 2 * q + fh;
            const f32x16& a = acc[half * 2 + m2][ni];
            const float sc = p.out_scale;
            buf[r * 16 + (ch ^ (r & 15))] = __builtin_bit_cast(
                u32x4, f32x4{a[4 * q] * sc, a[4 * q + 1] * sc, a[4 * q + 2] * sc, a[4 * q + 3] * sc});
          }
      }
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (0x3 << 14));  // lgkmcnt(0): own writes done
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int idx = it * 64 + lane;
        const int r = idx >> 4, c = idx & 15;
        const u32x4 v = buf[r * 16 + (c ^ (r & 15))];
        const int grow = tm * kBM + wm * (32 * MI) + half * 64 + r;
        if (grow < p.M)
          *reinterpret_cast<u32x4*>(C + static_cast<int64_t>(grow) * p.ldc + tn * BN + wn * 32 * NI + 4 * c) = v;
      }
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (0x3 << 14));  // reads done before the next pass
      __builtin_amdgcn_wave_barrier();
    }
  } else if (rin) {
    gemm_epilogue<BN, WM, WN, EPI, OP, TRANS, true>(p, acc, tm, tn, wm, wn, lane);
  } else {
    gemm_epilogue<BN, WM, WN, EPI, OP, TRANS, false, TA>(p, acc, tm, tn, wm, wn, lane);
  }
}

// Compute units of the current device (cached per device id).
inline int gemm_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// Rows of A in memory: M, or M rounded up to whole 16-row groups when A is tiled.
inline int64_t a_rows(const GemmParams& p) { return p.a_tiled ? (static_cast<int64_t>(p.M) + 15) & ~15 : p.M; }

// Preconditions of the tiled operands (each tiled matrix is dense: ld equals its row length;
// 16-row loads of tiled B stay inside one segment).
inline bool tiled_ok(const GemmParams& p, int epi) {
  if (p.a_tiled && p.lda != p.K) return false;
  if (p.b_tiled && (p.ldb != p.K || (epi != EPI_SWIGLU_16 && (p.nseg0 % 16 != 0 || p.nseg1 % 16 != 0))))
    return false;
  // a tiled SwiGLU output goes with a tiled A (one template flag), other outputs are row-major
  if (p.c_tiled && (epi != EPI_SWIGLU_16 || p.ldc != p.N / 2)) return false;
  if (epi == EPI_SWIGLU_16 && p.c_tiled != p.a_tiled) return false;
  return true;
}

// Buffer-descriptor loads address A and each B segment with 32-bit byte offsets, and one load
// instruction covers 16 consecutive B rows of a single segment. Q3_GEMM_ADDR64 (environment)
// forces the 64-bit address path, so that it can be tested at small sizes.
inline bool gemm_buffer_ok(const GemmParams& p, int epi) {
  if (!Q3_GEMM_BUF || std::getenv("Q3_GEMM_ADDR64") != nullptr) return false;
  const int64_t lim = 0x7fffffff;
  if (2 * a_rows(p) * p.lda > lim) return false;
  if (epi == EPI_SWIGLU_16) return 2 * static_cast<int64_t>(p.N / 2) * p.ldb <= lim;
  if (p.nseg0 % 16 != 0 || p.nseg1 % 16 != 0) return false;
  const int64_t rows = std::max<int64_t>(p.nseg0, std::max<int64_t>(p.nseg1 - p.nseg0, p.N - p.nseg1));
  return 2 * rows * p.ldb <= lim;
}



template <int BN, int WM, int WN, int EPI, int OP, bool CVT>
static hipError_t launch_t(const GemmParams& p, hipStream_t s) {
  const int tiles = ((p.M + kBM - 1) / kBM) * (p.N / BN);
  constexpr int NS = (Q3_GEMM_STAGES * (kBM + BN) * 64 + (BN % 128 ? 1024 : 0) <= 160 * 1024)
                         ? Q3_GEMM_STAGES : 4;
  // SwiGLU outputs with whole groups of NS K steps per tile: one workgroup per CU walks
  // several tiles (grid a multiple of 8, so a workgroup keeps the XCD its tiles map to). The
  // 16-bit store epilogue inside the loop pushed the QKV tiles past 256 registers (spills), so
  // those stay one tile per workgroup.
  int grid = tiles;
  if (EPI == EPI_SWIGLU_16 && (p.K / kBK2) % NS == 0 && Q3_GEMM_PERSIST) {
    const int cus = gemm_cu_count();
    if (cus >= 8 && tiles > cus) grid = cus & ~7;
  }
  auto go = [&](auto ta, auto tb) {
    constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
    if (gemm_buffer_ok(p, EPI))
      gemm_d2l_kernel<BN, WM, WN, EPI, OP, CVT, NS, true, false, TA, TB><<<grid, 64 * WM * WN, 0, s>>>(p);
    else
      gemm_d2l_kernel<BN, WM, WN, EPI, OP, CVT, NS, false, false, TA, TB><<<grid, 64 * WM * WN, 0, s>>>(p);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (p.b_tiled) {
    // tiled B is fp16 (no conversion)
    if constexpr (OP == OP_F16 && !CVT) {
      if (p.a_tiled) go(T_{}, T_{});
      else go(F_{}, T_{});
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    if (p.a_tiled) go(T_{}, F_{});
    else go(F_{}, F_{});
  }
  return hipGetLastError();
}

// Q4_0 weights decoded in the weight-tile path (A through buffer loads: the caller checks
// that its byte extent fits 32-bit offsets).
template <int BN, int WM, int WN, int EPI, int OP>
static hipError_t launch_q4(const GemmParams& p, hipStream_t s) {
  const int tiles = ((p.M + kBM - 1) / kBM) * (p.N / BN);
  constexpr int NS = 4;
  int grid = tiles;
  if (EPI == EPI_SWIGLU_16 && (p.K / kBK2) % NS == 0 && Q3_GEMM_PERSIST) {
    const int cus = gemm_cu_count();
    if (cus >= 8 && tiles > cus) grid = cus & ~7;
  }
  if (p.a_tiled)
    gemm_d2l_kernel<BN, WM, WN, EPI, OP, false, NS, true, true, true><<<grid, 64 * WM * WN, 0, s>>>(p);
  else
    gemm_d2l_kernel<BN, WM, WN, EPI, OP, false, NS, true, true, false><<<grid, 64 * WM * WN, 0, s>>>(p);
  return hipGetLastError();
}

template <int EPI, int OP>
static hipError_t launch_q4_nb(const GemmParams& p, int nb, hipStream_t s) {
  if (nb == 4) return launch_q4<256, 2, 4, EPI, OP>(p, s);
  if constexpr (EPI == EPI_SWIGLU_16) {
    return hipErrorInvalidValue;
  } else {
    if (nb == 3) return launch_q4<192, 4, 2, EPI, OP>(p, s);
    if (nb == 2) return launch_q4<128, 4, 2, EPI, OP>(p, s);
    return hipErrorInvalidValue;
  }
}


// nb selects the tile width 64*nb: 256 (8 waves, 2 x 4), 192 (8 waves, 4 x 2), 128 (8 waves, 4 x 2)
template <int EPI, int OP, bool CVT>
static hipError_t launch_nb(const GemmParams& p, int nb, hipStream_t s) {
  if (nb == 4) return launch_t<256, 2, 4, EPI, OP, CVT>(p, s);
  if constexpr (EPI == EPI_SWIGLU_16) {
    return hipErrorInvalidValue;
  } else {
    if (nb == 3) return launch_t<192, 4, 2, EPI, OP, CVT>(p, s);
    if (nb == 2) return launch_t<128, 4, 2, EPI, OP, CVT>(p, s);
    return hipErrorInvalidValue;
  }
}

template <int OP, bool CVT>
static hipError_t launch_epi(const GemmParams& p, int epi, int nb, hipStream_t s) {
  switch (epi) {
    case EPI_STORE_16: return launch_nb<EPI_STORE_16, OP, CVT>(p, nb, s);
    case EPI_STORE_F32: return launch_nb<EPI_STORE_F32, OP, CVT>(p, nb, s);
    case EPI_SWIGLU_16: return launch_nb<EPI_SWIGLU_16, OP, CVT>(p, nb, s);
    default: return hipErrorInvalidValue;
  }
}


// Instantiation units: each launches one operand family (the kernel templates above compile
// in separate translation units, in parallel).
hipError_t gemm_part_bf16(const GemmParams& p, int epi, int nb, hipStream_t s);      // bf16 A and B
hipError_t gemm_part_f16(const GemmParams& p, int epi, int nb, hipStream_t s);       // fp16 A and B
hipError_t gemm_part_f16_cvt(const GemmParams& p, int epi, int nb, hipStream_t s);   // fp16 A, bf16 B
hipError_t gemm_part_q4(const GemmParams& p, int epi, int op, int nb, hipStream_t s);  // Q4_0 B

}  // namespace q3
