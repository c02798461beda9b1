// Grouped-query flash attention, 16-bit (fp16 or bf16) operands, head_dim 64 or 128, for gfx950.
//
// Causal: o[s, h] = sum_{j<=s} softmax_j(scale * q[s,h] . k[j,g]) v[j,g] with
// g = h / (nh / nkv) (cortiq-engine 0.8.21, qwen3te.rs: the per-pair causal loop and
// `attention_gemm`; hf2q 0.1.1, qwen3vl_text/forward.rs: SDPA causal, scale 1/sqrt(head_dim)).
// Bidirectional (a runtime flag): every key j < S (inferencelayer 0.2.3, vision.rs, the vision
// block's `attention`; cortiq-engine 0.8.51, onevision2.rs, `attend`).
// Unlike those pages, no score matrix is formed: keys stream through LDS in tiles of 64 and
// each query row keeps an online softmax (running maximum and sum, fp32, base 2).
//
// Work split. A workgroup of 8 waves owns one KV head g and a block of tokens; its waves
// cover all G = nh/nkv query heads of g for that block (32 tokens per wave), so every K/V
// tile brought into LDS serves the whole GQA group. Workgroups with the most keys (the last
// token blocks) are dispatched first, and with nkv = 8 the workgroups of one KV head land on
// one XCD (ids congruent mod 8), so that head's K/V stays in that XCD's L2.
//
// Per wave and 64-key tile, with v_mfma_f32_32x32x16_{f16,bf16}:
//   S^T = K Q^T     (A = K from LDS, B = Q^T held in registers)  -> lane l holds query row
//                   l%32 and 16 of the 32 keys of each 32-key block, so the row maximum
//                   needs one cross-lane exchange (lanes l and l^32, v_permlane32_swap);
//   O^T += V^T P^T  (A = V^T from a transposed LDS copy, B = P^T straight from the S^T
//                   accumulators converted to 16 bits) -> lane l keeps query row l%32 of the
//                   output, so the rescale by exp2(m_old - m_new) and the final 1/sum are
//                   lane-local. The K index of this product enumerates the tile's keys in the
//                   order the S^T accumulators hold them; V^T is read in that same order.
//
// Software pipelining. On CDNA the MFMA unit and the VALU overlap well within one wave's
// instruction stream and much less across the two waves of a SIMD, so every wave overlaps
// its own MFMAs with its own softmax arithmetic. Iteration t, one barrier per iteration:
//   A  S^T(t) = K(t) Q^T                  || P(t-1) = exp2(S(t-1) c - m), row sums, packing
//   B  O^T += V^T(t-1) P^T(t-1)           || row maxima of S(t) (after the causal mask)
//   C  running maximum update; O and the sums rescaled when a row's maximum passed it (fp16:
//      by more than 8 in log2 units, lazy rescaling)
// S(t) and S(t-1) live in two register sets that swap roles every iteration.
//
// LDS: K and V^T tiles, two slots each. Rows are padded instead of XOR-swizzled, so every
// fragment address is a per-lane base plus a compile-time offset:
//   K   [64 keys][17 x 16 B]  16 chunks of 8 hd + 1 pad; a 16-lane read of one chunk column
//                             touches 16 distinct 16-byte bank groups;
//   V^T [128 hd][18 x 8 B]    16 granules of 4 keys + 2 pad. Within each 32-key block the
//                             granules are stored in the order 0,2,1,3,4,6,5,7, so the two
//                             granules an MFMA lane needs (4-key groups i and i+2 of the S^T
//                             accumulator order) are adjacent: one 16-byte read.
// Waves 0-3 stage K tiles, waves 4-7 V tiles (transposed on the way into LDS). Iteration t
// writes K(t+1) and V(t) to LDS at its end, into slots last read in iteration t-1; their global
// loads were issued one iteration earlier (K(t+2) and V(t+1) are requested at the top of
// iteration t), into two register sets that alternate, so a load has a whole iteration to land.
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "kernels.h"

// Exponent-offset slack (log2 units) for fp16 operands: the running maximum (and with it the
// rescale of O and of the row sums) moves only when a row's maximum exceeds it by more than
// this, so after the first tiles almost no tile pays for a rescale. Probabilities then reach up
// to 2^8 before packing to fp16 (11-bit significand at any magnitude); the largest one is no
// longer exactly 1, which fp16 absorbs but bf16's 8-bit significand does not, so bf16 operands
// rescale on every increase.
#ifndef Q3_ATTN_LAZY
#define Q3_ATTN_LAZY 8
#endif

namespace q3 {

constexpr int kKT = 64;    // keys per tile
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kVRow = 18;  // u32x2 per padded V^T row (16 granules of 4 keys + 2 pad)

// position of 4-key granule gi (0..15 within the tile) in a V^T row: 4h+2x+s -> 4h+2s+x
__device__ __forceinline__ int vt_pos(int gi) {
  return (gi & 12) | ((gi & 1) << 1) | ((gi >> 1) & 1);
}

// max(x[l], x[l ^ 32]) for every lane l: v_permlane32_swap exchanges the two lane halves
// between its two operands, so the pair it returns holds x[l] and x[l ^ 32] in some order
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int G, int OP, bool BUF, int HD>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const AttnParams p) {
  using F = Fmt<OP>;
  constexpr int NB = 8 / G;
  constexpr int TOK = 32 * NB;
  constexpr int NKS = HD / 16;     // 16-wide K steps of the S^T product
  constexpr int ND = HD / 32;      // 32-row blocks of O^T
  constexpr int NCH = HD / 8;      // 16-byte chunks per K / V row
  constexpr int KROW = NCH + 1;    // u32x4 per padded K row
  constexpr int KPT = kKT * NCH / 256;  // K chunks staged per K-loader thread
  __shared__ __attribute__((aligned(16))) u32x4 Ks[2][kKT * KROW];
  __shared__ __attribute__((aligned(16))) u32x2 Vts[2][HD * kVRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nblk = (p.S + TOK - 1) / TOK;
  const int g = blockIdx.x % p.nkv;
  const int blk = nblk - 1 - blockIdx.x / p.nkv;
  const int t0 = blk * TOK;
  const int qrow = lane & 31;
  const int hi = lane >> 5;
  const int bt = wave % NB, hl = wave / NB;
  const int hq = g * G + hl;
  const int my_t = t0 + 32 * bt + qrow;
  // causal: keys up to the row's own token; bidirectional: every key of the sequence
  const bool causal = p.causal != 0;
  const int lim = causal ? min(my_t, p.S - 1) : p.S - 1;
  const int ntiles = ((causal ? min(p.S, t0 + TOK) : p.S) + kKT - 1) / kKT;

  u32x4 qf[NKS];
  {
    const bool ok = my_t < p.S;
    const uint16_t* qp = p.q + static_cast<int64_t>(ok ? my_t : 0) * p.q_stride + hq * HD + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      if (!ok) v = u32x4{0, 0, 0, 0};
      qf[ks] = v;
    }
  }

  f32x16 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  f32x16 sa[2], sb[2];
  u32x4 pf[4];
  float m_run = -INFINITY;
  float l_part = 0.f;

  // staging: waves 0-3 carry K chunks tv + 256 i; waves 4-7 carry hd chunk vc of keys 4vg..+3
  const bool k_loader = wave < 4;  // wave-uniform (the buffer descriptor depends on it)
  const int tv = tid & 255;
  const int vg = tv & 15, vc = tv >> 4;
  const bool v_active = vc < NCH;  // with HD = 64 waves 6 and 7 stage nothing (wave-uniform)
  const int vpos = vt_pos(vg);
  // staging registers of the global loads, two sets: K(j) goes to set j % 2 and V(j) to set
  // (j + 1) % 2 (so both roles request into, and store from, the same set in an iteration), and
  // each is written to LDS one iteration after it was requested
  u32x4 st0[4], st1[4];
  static_assert(KPT <= 4, "head_dim");
  // K / V rows come in through buffer loads when the operand's byte extent fits the 32-bit
  // range (BUF), with a per-lane 32-bit byte offset, so the loop carries no 64-bit address
  // arithmetic; otherwise through 64-bit addresses. Either way a row index at or past S is
  // clamped to S - 1: such keys are masked (probability 0) and their values are finite data
  // of the sequence, so nothing past the last row is read and no 0 * Inf/NaN can reach O.
  const int64_t row_elems = k_loader ? p.k_stride : p.v_stride;
  const uint16_t* gbase = (k_loader ? p.k : p.v) + g * HD;
  int trow[4], tcol[4];  // row within the tile and element column of this thread's chunks
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tv + 256 * i;
    trow[i] = k_loader ? c / NCH : 4 * vg + i;
    tcol[i] = k_loader ? (c % NCH) * 8 : (v_active ? vc : 0) * 8;
  }
  const int nst = k_loader ? KPT : (v_active ? 4 : 0);  // this thread's staged chunks (uniform per wave)
  const int row_bytes = static_cast<int>(2 * row_elems);  // used only when BUF
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(gbase), static_cast<short>(0), p.S * row_bytes, 0x00020000);
  auto gload = [&](int tile, u32x4 (&st)[4]) __attribute__((always_inline)) {
    if constexpr (BUF) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nst) {
          const int row = min(tile * kKT + trow[i], p.S - 1);
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, row * row_bytes + 2 * tcol[i], 0, 0);
          st[i] = u32x4{v[0], v[1], v[2], v[3]};
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nst) {
          const int row = min(tile * kKT + trow[i], p.S - 1);
          st[i] = *reinterpret_cast<const u32x4*>(gbase + row * row_elems + tcol[i]);
        }
      }
    }
  };
  auto lstore = [&](int tile, const u32x4 (&st)[4]) __attribute__((always_inline)) {
    if (k_loader) {
      u32x4* dst = Ks[tile & 1];
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int c = tv + 256 * i;
        dst[(c / NCH) * KROW + (c % NCH)] = st[i];
      }
    } else if (v_active) {
      u32x2* dst = Vts[tile & 1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        dst[(vc * 8 + e) * kVRow + vpos] =
            u32x2{__builtin_amdgcn_perm(st[1][w], st[0][w], sel), __builtin_amdgcn_perm(st[3][w], st[2][w], sel)};
      }
    }
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (0x3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int kbase = qrow * KROW + hi;
  const int vbase = qrow * kVRow + 2 * hi;

  // P = exp2(S c - m), packed to 16 bits for the PV product; the row sum is taken over the
  // packed values (one v_dot2 per pair), i.e. over exactly the P that multiplies V.
  auto exp_part = [&](f32x16 (&sp)[2]) {
    const float neg_m = -m_run;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) sp[b][e] = fast_exp2(fmaf(sp[b][e], p.scale_log2, neg_m));
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st16 = 0; st16 < 4; ++st16) {
      const int b = st16 >> 1, half = st16 & 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[st16][e] = F::pack2(sp[b][half * 8 + 2 * e], sp[b][half * 8 + 2 * e + 1]);
        ls[e] = F::sum2(pf[st16][e], ls[e]);
      }
    }
    l_part += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  auto pv_all = [&](int tile) {
    const u32x2* vp = Vts[tile & 1] + vbase;
#pragma unroll
    for (int i = 0; i < 4 * ND; ++i) {
      const int st16 = i / ND, d = i % ND, b = st16 >> 1, half = st16 & 1;
      const u32x4 vv = *reinterpret_cast<const u32x4*>(vp + d * 32 * kVRow + 8 * b + 4 * half);
      o[d] = F::mfma(vv, pf[st16], o[d]);
    }
  };

  // one iteration: tile t into sc; sp holds S(t-1) (unless first)
  // stT: set t % 2 (requests of this iteration), stO: set (t + 1) % 2 (stored this iteration)
  auto iter = [&](int t, f32x16 (&sc)[2], f32x16 (&sp)[2], auto first, u32x4 (&stT)[4], u32x4 (&stO)[4])
      __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first)::value;
    const int kb = t * kKT;
    const bool next = t + 1 < ntiles;
    // K loaders request K(t+2) (written to LDS at the end of iteration t+1), V loaders V(t+1)
    const bool req = k_loader ? t + 2 < ntiles : next;
    if (req) gload(k_loader ? t + 2 : t + 1, stT);
    // A
    const u32x4* kp = Ks[t & 1] + kbase;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[b][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int b = 0; b < 2; ++b) sc[b] = F::mfma(kp[b * 32 * KROW + 2 * ks], qf[ks], sc[b]);
    if (!FIRST) {
      exp_part(sp);
      // anchor P^T here, so that the exponentials are scheduled among the S^T MFMAs above
      // instead of being sunk past the mask branch
#pragma unroll
      for (int st16 = 0; st16 < 4; ++st16) asm volatile("" ::"v"(pf[st16]));
    }
    // mask on diagonal (causal) and tail tiles (wave-uniform branch)
    if ((causal && kb + kKT - 1 > t0 + 32 * bt) || kb + kKT > p.S) {
      asm volatile("");
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb + b * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
          sc[b][e] = key > lim ? -INFINITY : sc[b][e];
        }
    }
    // B
    if (!FIRST) pv_all(t - 1);
    float mt = sc[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sc[b][e]);
    mt = max_halves(mt) * p.scale_log2;
    // C
    if (__builtin_amdgcn_ballot_w64(mt > m_run + (OP == OP_F16 ? static_cast<float>(Q3_ATTN_LAZY) : 0.f))) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
      m_run = m_new;
    }
    // stage K(t+1) / V(t), requested one iteration ago; this iteration's requests may still be
    // in flight (vmcnt counts them: KPT or 4 per thread)
    if (!req) {
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
    } else if (k_loader) {
      __builtin_amdgcn_s_waitcnt(KPT | (0x7 << 4) | (0xF << 8));
    } else {
      __builtin_amdgcn_s_waitcnt(4 | (0x7 << 4) | (0xF << 8));
    }
    if (!k_loader || next) lstore(k_loader ? t + 1 : t, stO);
    barrier();
  };

  // prologue: K(0) into LDS, K(1) and V(0) requested
  if (k_loader) {
    gload(0, st0);
    lstore(0, st0);
    if (ntiles > 1) gload(1, st1);
  } else {
    gload(0, st1);
  }
  barrier();

  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  iter(0, sa, sb, T_{}, st0, st1);
  int t = 1;
  for (; t + 1 < ntiles; t += 2) {
    iter(t, sb, sa, F_{}, st1, st0);
    iter(t + 1, sa, sb, F_{}, st0, st1);
  }
  if (t < ntiles) {
    iter(t, sb, sa, F_{}, st1, st0);
    exp_part(sb);
  } else {
    exp_part(sa);
  }
  pv_all(ntiles - 1);

  const float l_run = l_part + __shfl_xor(l_part, 32);
  if (my_t < p.S) {
    const float inv = 1.0f / l_run;
    // row-major: column hq*HD + 32d + j at row offset + hq*HD + 32d + j; tiled (16-row groups of
    // 32-column tiles): the row's offset inside its group, + 512 per 32 columns
    const int64_t o_row = p.o_tiled ? static_cast<int64_t>(my_t >> 4) * 16 * p.o_stride + (my_t & 15) * 32
                                    : static_cast<int64_t>(my_t) * p.o_stride;
    const int d_ks = p.o_tiled ? 512 : 32;
    uint16_t* op = p.o + o_row + (hq * HD / 32) * d_ks;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int j = 8 * q4 + 4 * hi;
        u32x2 w;
        w[0] = F::pack2(o[d][4 * q4 + 0] * inv, o[d][4 * q4 + 1] * inv);
        w[1] = F::pack2(o[d][4 * q4 + 2] * inv, o[d][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d * d_ks + j) = w;
      }
  }
}

template <int G, int OP, int HD>
static hipError_t launch_g(const AttnParams& p, hipStream_t s) {
  constexpr int TOK = 32 * kAttnWaves / G;
  const int nblk = (p.S + TOK - 1) / TOK;
  // Buffer loads address K and V with 32-bit byte offsets from the head's column (rows
  // clamped to S - 1). Q3_ATTN_ADDR64 (environment) forces the 64-bit address path, so that it
  // can be tested at small sizes.
  const int64_t extent = 2 * static_cast<int64_t>(p.S) * (p.k_stride > p.v_stride ? p.k_stride : p.v_stride);
  if (extent <= 0x7fffffff && std::getenv("Q3_ATTN_ADDR64") == nullptr)
    attn_fwd_kernel<G, OP, true, HD><<<nblk * p.nkv, kAttnThreads, 0, s>>>(p);
  else
    attn_fwd_kernel<G, OP, false, HD><<<nblk * p.nkv, kAttnThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <int OP, int HD>
static hipError_t launch_op(const AttnParams& p, hipStream_t s) {
  switch (p.nh / p.nkv) {
    case 1: return launch_g<1, OP, HD>(p, s);
    case 2: return launch_g<2, OP, HD>(p, s);
    case 4: return launch_g<4, OP, HD>(p, s);
    case 8: return launch_g<8, OP, HD>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_mfma(const AttnParams& p, int op, hipStream_t s) {
  if (p.S <= 0) return hipSuccess;
  if (p.nkv <= 0 || p.nh % p.nkv != 0) return hipErrorInvalidValue;
  if (p.o_tiled && p.o_stride != static_cast<int64_t>(p.nh) * p.head_dim) return hipErrorInvalidValue;
  if (p.head_dim == 128) {
    if (op == OP_BF16) return launch_op<OP_BF16, 128>(p, s);
    if (op == OP_F16) return launch_op<OP_F16, 128>(p, s);
  } else if (p.head_dim == 64) {
    if (op == OP_BF16) return launch_op<OP_BF16, 64>(p, s);
    if (op == OP_F16) return launch_op<OP_F16, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace q3
