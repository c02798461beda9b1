// Causal grouped-query flash attention, 16-bit (fp16 or bf16) operands, head_dim 128, for gfx950.
//
// Computes o[s, h] = sum_{j<=s} softmax_j(scale * q[s,h] . k[j,g]) v[j,g] with
// g = h / (nh / nkv) (cortiq-engine 0.8.21, qwen3te.rs: the per-pair causal loop and
// `attention_gemm`; hf2q 0.1.1, qwen3vl_text/forward.rs: SDPA causal, scale 1/sqrt(head_dim)).
// Unlike those pages, no score matrix is formed: keys stream through LDS in tiles of 64 and
// each query row keeps an online softmax (running maximum and sum, fp32, base 2).
//
// Work split. A workgroup of 8 waves owns one KV head g and a block of tokens; its waves
// cover all G = nh/nkv query heads of g for that block (32 tokens per wave), so every K/V
// tile brought into LDS serves the whole GQA group. Workgroups with the most keys (the last
// token blocks) are dispatched first, and with nkv = 8 the workgroups of one KV head land on
// one XCD (ids congruent mod 8), so that head's K/V stays in that XCD's L2.
//
// Per wave and 64-key tile, with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T     (A = K from LDS, B = Q^T held in registers)  -> lane l holds query row
//                   l%32 and 16 of the 32 keys of each 32-key block, so the row maximum and
//                   sum need one cross-lane exchange (lanes l and l^32);
//   O^T += V^T P^T  (A = V^T from a transposed LDS copy, B = P^T straight from the S^T
//                   accumulators converted to bf16) -> lane l keeps query row l%32 of the
//                   output, so the rescale by exp2(m_old - m_new) and the final 1/sum are
//                   lane-local. The K index of this product enumerates the tile's keys in the
//                   order the S^T accumulators hold them; V^T is read in that same order.
#include "common.h"
#include "kernels.h"

#ifndef Q3_ATTN_LAZY
#define Q3_ATTN_LAZY 0
#endif

namespace q3 {

constexpr int kHD = 128;
constexpr int kKT = 64;          // keys per tile
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;

// K tile in LDS: [64 keys][16 chunks of 8 hd], chunk index XOR-swizzled by key.
__device__ __forceinline__ int swz_k(int key) { return key & 15; }
// V^T tile in LDS: [128 hd][16 granules of 4 keys], granule index XOR-swizzled by hd row.
__device__ __forceinline__ int swz_v(int hd) { return (hd ^ (hd >> 4)) & 15; }

template <int G, int OP>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const AttnParams p) {
  using F = Fmt<OP>;
  constexpr int TOK = 32 * kAttnWaves / G;  // tokens per workgroup
  __shared__ u32x4 Ks[2][kKT * 16];
  __shared__ u32x2 Vts[2][kHD * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform by construction
  const int nblk = (p.S + TOK - 1) / TOK;
  const int g = blockIdx.x % p.nkv;
  const int blk = nblk - 1 - blockIdx.x / p.nkv;
  const int t0 = blk * TOK;
  const int hq = g * G + wave % G;
  const int wt0 = t0 + (wave / G) * 32;  // this wave's first query token
  const int qrow = lane & 31;
  const int hi = lane >> 5;
  const int my_t = wt0 + qrow;

  // Q^T operand: lane holds q[my_t, hq, 16*ks + 8*hi .. +8] for ks = 0..7.
  u32x4 qf[8];
  {
    const bool ok = my_t < p.S;
    const uint16_t* qp = p.q + static_cast<int64_t>(ok ? my_t : 0) * p.q_stride + hq * kHD + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      if (!ok) v = u32x4{0, 0, 0, 0};
      qf[ks] = v;
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  float m_run = -INFINITY;  // exponent offset: running max of scaled scores (base 2)
  float l_run = 0.f;

  const int wg_end = min(p.S, t0 + TOK);        // keys this workgroup needs
  const int wave_end = min(p.S, wt0 + 32);      // keys this wave needs
  const bool wave_live = wt0 < p.S;
  const int ntiles = (wg_end + kKT - 1) / kKT;

  // Global -> register staging. Waves 0-3 fetch K (4 chunks of 16 B each), waves 4-7 fetch
  // V as 4 consecutive keys x 8 hd values per thread, to be written transposed.
  const bool k_loader = tid < 256;
  const int lt = tid & 255;
  u32x4 st[4];
  auto gload = [&](int kb) {
    if (k_loader) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = lt + 256 * i;
        const int key = min(kb + (c >> 4), p.S - 1);
        st[i] = *reinterpret_cast<const u32x4*>(p.k + static_cast<int64_t>(key) * p.k_stride +
                                                 g * kHD + (c & 15) * 8);
      }
    } else {
      const int kg = lt >> 4, hc = lt & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = min(kb + 4 * kg + r, p.S - 1);
        st[r] = *reinterpret_cast<const u32x4*>(p.v + static_cast<int64_t>(key) * p.v_stride +
                                                 g * kHD + hc * 8);
      }
    }
  };
  auto lstore = [&](int buf) {
    if (k_loader) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = lt + 256 * i;
        const int key = c >> 4;
        Ks[buf][key * 16 + ((c & 15) ^ swz_k(key))] = st[i];
      }
    } else {
      const int kg = lt >> 4, hc = lt & 15;
      // st[r] holds v[key 4kg+r][hd 8hc .. 8hc+7] as 4 words of two 16-bit values each; the
      // granule for hd row 8hc+e gathers the e-th value of the four keys (byte permutes).
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const int hd = hc * 8 + e;
        Vts[buf][hd * 16 + (kg ^ swz_v(hd))] =
            u32x2{__builtin_amdgcn_perm(st[1][w], st[0][w], sel), __builtin_amdgcn_perm(st[3][w], st[2][w], sel)};
      }
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int kb = it * kKT;
    const bool more = it + 1 < ntiles;
    if (more) gload(kb + kKT);

    if (wave_live && kb < wave_end) {
      // ---- S^T = K Q^T for two 32-key blocks (the two accumulation chains interleaved)
      f32x16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[b][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int ch = 2 * ks + hi;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int key = b * 32 + qrow;
          s[b] = F::mfma(Ks[buf][key * 16 + (ch ^ swz_k(key))], qf[ks], s[b]);
        }
      }
      // ---- causal mask, online softmax (base 2). The exponent offset m_run moves only when a
      // row's maximum exceeds it by more than Q3_ATTN_LAZY (then O and the running sum are
      // rescaled, skipped for the whole wave when no row needs it); probabilities formed
      // against a stale offset stay below 2^Q3_ATTN_LAZY, so the 16-bit P operand cannot
      // overflow. The result is the same softmax: numerator and denominator share the offset.
      // With 0 the row maximum's probability is exactly 1, the most precise choice.
      if (kb + kKT - 1 > wt0 || kb + kKT > p.S) {  // wave-uniform: only diagonal / tail tiles
        const int lim = min(my_t, p.S - 1);          // last live key of this lane's row
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb + b * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
            s[b][e] = key > lim ? -INFINITY : s[b][e];
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s[b][e]);
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * p.scale_log2;  // scaled row maximum of this tile
      if (__builtin_amdgcn_ballot_w64(mt > m_run + static_cast<float>(Q3_ATTN_LAZY))) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
        m_run = m_new;
      }
      const float neg_m = -m_run;
      float ls = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pe = fast_exp2(fmaf(s[b][e], p.scale_log2, neg_m));
          s[b][e] = pe;
          ls += pe;
        }
      l_run += ls + __shfl_xor(ls, 32);

      // ---- O^T += V^T P^T, four 16-key steps
#pragma unroll
      for (int st16 = 0; st16 < 4; ++st16) {
        const int b = st16 >> 1, half = st16 & 1;
        u32x4 pf;
#pragma unroll
        for (int e = 0; e < 4; ++e) pf[e] = F::pack2(s[b][half * 8 + 2 * e], s[b][half * 8 + 2 * e + 1]);
        // this lane's 8 K-slots are keys 32b + 16half + 4hi + {0..3} and the same + 8
        const int gA = (b * 32 + half * 16) / 4 + hi;
        const int gB = gA + 2;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int hd = d * 32 + qrow;
          const u32x2 lo = Vts[buf][hd * 16 + (gA ^ swz_v(hd))];
          const u32x2 hi2 = Vts[buf][hd * 16 + (gB ^ swz_v(hd))];
          const u32x4 vv = {lo[0], lo[1], hi2[0], hi2[1]};
          o[d] = F::mfma(vv, pf, o[d]);
        }
      }
    }

    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

  if (wave_live && my_t < p.S) {
    const float inv = 1.0f / l_run;
    uint16_t* op = p.o + static_cast<int64_t>(my_t) * p.o_stride + hq * kHD;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // elements e = 4*q4 .. 4*q4+3 are hd rows d*32 + 8*q4 + 4*hi + 0..3
        const int hd0 = d * 32 + 8 * q4 + 4 * hi;
        u32x2 w;
        w[0] = F::pack2(o[d][4 * q4 + 0] * inv, o[d][4 * q4 + 1] * inv);
        w[1] = F::pack2(o[d][4 * q4 + 2] * inv, o[d][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + hd0) = w;
      }
  }
}

template <int G, int OP>
static hipError_t launch_g(const AttnParams& p, hipStream_t s) {
  constexpr int TOK = 32 * kAttnWaves / G;
  const int nblk = (p.S + TOK - 1) / TOK;
  attn_fwd_kernel<G, OP><<<nblk * p.nkv, kAttnThreads, 0, s>>>(p);
  return hipGetLastError();
}

template <int OP>
static hipError_t launch_op(const AttnParams& p, hipStream_t s) {
  switch (p.nh / p.nkv) {
    case 1: return launch_g<1, OP>(p, s);
    case 2: return launch_g<2, OP>(p, s);
    case 4: return launch_g<4, OP>(p, s);
    case 8: return launch_g<8, OP>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_mfma(const AttnParams& p, int op, hipStream_t s) {
  if (p.S <= 0) return hipSuccess;
  if (p.nkv <= 0 || p.nh % p.nkv != 0) return hipErrorInvalidValue;
  if (op == OP_BF16) return launch_op<OP_BF16>(p, s);
  if (op == OP_F16) return launch_op<OP_F16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace q3
