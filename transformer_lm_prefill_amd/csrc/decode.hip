// The key/value cache a prefill leaves behind and one decode step of the layer (hf2q 0.1.1,
// qwen3vl_text/forward.rs, module doc: the KV cache for incremental decode that the prefill-only
// path defers).
//
// Cache layout: per layer, K and V each [n_kv_heads][capacity][head_dim] in the layer's operand
// type. Head-major, so one KV head's keys form one contiguous [capacity, hd] matrix that a
// decode step streams with whole-line loads; the prefill writes rows 0..S-1 of every head, a
// decode step appends its row.
//
// Decode attention (one query token per step) is HBM-bound: every cached key and value is read
// once per step and used by the nh/nkv query heads of its group. It is split over the keys:
// workgroup (split, kv head) walks 64-key tiles. Each tile's K and V go through LDS (coalesced
// 16-byte loads, the next tile's loads in flight while the current one is scored); lane j of a
// wave scores key j against one query head (query rows read from LDS as broadcasts; v_dot2 with
// fp32 accumulation for 16-bit caches), keeps a base-2 online softmax, and then every lane
// accumulates two output elements over the tile's keys with the probabilities broadcast from
// LDS. Each (head, split) leaves (max, sum, o) in the workspace; a second kernel merges the
// splits.
//
// Decode projections are matrix-vector products: the weights stream once with 16-byte loads,
// four rows per wave, the input vector from L2; epilogues fuse the residual add and SwiGLU.
#include "common.h"
#include "kernels.h"

namespace q3 {

// ---- cache write -------------------------------------------------------------------------------
// Thread = 8 consecutive elements of one (token, kv head) row; blockIdx.y: 0 = K, 1 = V.
template <int SDT, int CDT>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(KvWriteParams p) {
  const int chunks = p.hd / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(p.n) * p.nkv * chunks) return;
  const int c = static_cast<int>(idx % chunks);
  const int64_t rest = idx / chunks;
  const int g = static_cast<int>(rest % p.nkv);
  const int64_t t = rest / p.nkv;
  const bool is_v = blockIdx.y != 0;
  const void* src = is_v ? p.v : p.k;
  void* dst = is_v ? p.vc : p.kc;
  const int64_t si = t * (is_v ? p.v_stride : p.k_stride) + static_cast<int64_t>(g) * p.hd + c * 8;
  const int64_t di = (static_cast<int64_t>(g) * p.capacity + p.row0 + t) * p.hd + c * 8;
  if (SDT == CDT && SDT != DT_F32) {
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + di) =
        *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + si);
  } else {
    float v[8];
    load8<SDT>(src, si, v);
    store8<CDT>(dst, di, v);
  }
}

template <int SDT>
static hipError_t kv_write_cdt(const KvWriteParams& p, int cdt, dim3 grid, hipStream_t s) {
  if (cdt == DT_F16) kv_cache_write_kernel<SDT, DT_F16><<<grid, 256, 0, s>>>(p);
  else if (cdt == DT_BF16) kv_cache_write_kernel<SDT, DT_BF16><<<grid, 256, 0, s>>>(p);
  else if (cdt == DT_F32) kv_cache_write_kernel<SDT, DT_F32><<<grid, 256, 0, s>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_kv_cache_write(const KvWriteParams& p, int src_dt, int cache_dt, hipStream_t s) {
  if (p.n <= 0) return hipSuccess;
  if (p.hd % 8 != 0) return hipErrorInvalidValue;
  const int64_t threads = static_cast<int64_t>(p.n) * p.nkv * (p.hd / 8);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256), 2);
  if (src_dt == DT_F16) return kv_write_cdt<DT_F16>(p, cache_dt, grid, s);
  if (src_dt == DT_BF16) return kv_write_cdt<DT_BF16>(p, cache_dt, grid, s);
  if (src_dt == DT_F32) return kv_write_cdt<DT_F32>(p, cache_dt, grid, s);
  return hipErrorInvalidValue;
}

// ---- decode attention ------------------------------------------------------------------------
// workgroups the key splits of one decode-attention call aim at (256 and 1024 measured slower
// at 16k-32k keys, equal at 4k)
constexpr int kDecWorkgroups = 512;
constexpr int kDecTile = 64;       // keys per tile
constexpr int kDecMaxGroup = 16;   // query heads per KV head (4 per wave)

int decode_tiles_per_split(int len, int nkv) {
  const int ntiles = (len + kDecTile - 1) / kDecTile;
  const int target = nkv >= kDecWorkgroups ? 1 : kDecWorkgroups / nkv;
  return (ntiles + target - 1) / target;
}

int decode_max_splits(int len, int nkv) {
  const int ntiles = (len + kDecTile - 1) / kDecTile;
  const int target = nkv >= kDecWorkgroups ? 1 : kDecWorkgroups / nkv;
  return ntiles < target ? ntiles : target;
}

int decode_num_splits(int len, int nkv) {
  const int ntiles = (len + kDecTile - 1) / kDecTile;
  const int tps = decode_tiles_per_split(len, nkv);
  return (ntiles + tps - 1) / tps;
}

// Dot product of one 16-byte chunk of a key row with the same chunk of a query row, added to
// acc. (Each vector element is copied to a scalar before the bit cast: a bit cast of a vector
// element expression reads the vector's first element with this compiler.)
template <int CDT>
__device__ __forceinline__ float dot_chunk(u32x4 k, u32x4 q, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t kw = k[e], qw = q[e];
    if (CDT == DT_F32) {
      acc = fmaf(__uint_as_float(kw), __uint_as_float(qw), acc);
    } else if (CDT == DT_F16) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, kw), __builtin_bit_cast(h2, qw), acc, false);
    } else {
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw), __builtin_bit_cast(bf16x2, qw), acc,
                                            false);
    }
  }
  return acc;
}

template <int CDT, int HD>
__global__ __launch_bounds__(256) void decode_attn_partial_kernel(DecodeAttnParams p) {
  constexpr int ES = CDT == DT_F32 ? 4 : 2;
  constexpr int ROWB = HD * ES + 16;            // padded LDS row: 16-lane groups hit distinct banks
  constexpr int CH = HD * ES / 16;              // 16-byte chunks per row
  constexpr int LOADS = kDecTile * CH / 256;    // 16-byte loads per thread per matrix per tile
  constexpr int LPK = HD / 2;                   // P·V: lanes per key, two output elements each
  constexpr int KPS = 64 / LPK;                 // keys per step (1 at hd 128, 2 at hd 64)
  constexpr int RUN = kDecTile / KPS;           // probabilities one lane consumes per tile
  __shared__ __align__(16) char ks[kDecTile * ROWB];
  __shared__ __align__(16) char vs[kDecTile * ROWB];
  __shared__ __align__(16) char qs[kDecMaxGroup * HD * ES];
  __shared__ __align__(16) float pb[4][kDecTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.y, split = blockIdx.x;
  const int G = p.nh / p.nkv;
  const int ntiles = (p.len + kDecTile - 1) / kDecTile;
  const int t0 = split * p.tiles_per_split;
  const int t1 = min(ntiles, t0 + p.tiles_per_split);

  const char* kbase = static_cast<const char*>(p.kc) + static_cast<int64_t>(g) * p.capacity * HD * ES;
  const char* vbase = static_cast<const char*>(p.vc) + static_cast<int64_t>(g) * p.capacity * HD * ES;
  u32x4 kr[LOADS], vr[LOADS];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int i = tid + 256 * r;
      const int key = min(t * kDecTile + i / CH, p.len - 1);  // rows past the end repeat the last
      const int64_t off = static_cast<int64_t>(key) * HD * ES + (i % CH) * 16;
      kr[r] = *reinterpret_cast<const u32x4*>(kbase + off);
      vr[r] = *reinterpret_cast<const u32x4*>(vbase + off);
    }
  };

  const int nhw = (G - wave + 3) / 4;  // this wave's heads: wave, wave + 4, ... < G
  float m[4], lsum[4], o0[4], o1[4];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    m[hh] = -INFINITY;
    lsum[hh] = 0.f;
    o0[hh] = 0.f;
    o1[hh] = 0.f;
  }
  const int sub = lane / LPK, d0 = 2 * (lane % LPK);

  // the group's query rows (at most kDecMaxGroup * HD values, QPT per thread) are requested
  // first and the first tile's K / V rows right after, so the two latencies overlap; the rows go
  // to LDS in the cache's format (16-bit: rounded to nearest even)
  constexpr int QPT = kDecMaxGroup * HD / 256;
  float qv[QPT];
#pragma unroll
  for (int r = 0; r < QPT; ++r) {
    const int i = tid + 256 * r;
    qv[r] = p.q[static_cast<int64_t>(g) * G * HD + min(i, G * HD - 1)];  // (only i < G * HD is kept)
  }
  asm volatile("" ::: "memory");  // the query requests go out first,
  if (t0 < t1) load_tile(t0);
  asm volatile("" ::: "memory");  // and their stores (with the wait) come after the tile requests
#pragma unroll
  for (int r = 0; r < QPT; ++r) {
    const int i = tid + 256 * r;
    if (i < G * HD) {
      if (CDT == DT_F32) reinterpret_cast<float*>(qs)[i] = qv[r];
      else reinterpret_cast<uint16_t*>(qs)[i] = CDT == DT_BF16 ? f2bf(qv[r]) : f2h(qv[r]);
    }
  }
  for (int t = t0; t < t1; ++t) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int i = tid + 256 * r;
      *reinterpret_cast<u32x4*>(ks + (i / CH) * ROWB + (i % CH) * 16) = kr[r];
      *reinterpret_cast<u32x4*>(vs + (i / CH) * ROWB + (i % CH) * 16) = vr[r];
    }
    __syncthreads();
    if (t + 1 < t1) load_tile(t + 1);
    const bool valid = t * kDecTile + lane < p.len;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      if (hh >= nhw) break;
      const int h = wave + 4 * hh;
      float sc = 0.f;
#pragma unroll 4
      for (int c = 0; c < CH; ++c)
        sc = dot_chunk<CDT>(*reinterpret_cast<const u32x4*>(ks + lane * ROWB + c * 16),
                            *reinterpret_cast<const u32x4*>(qs + h * HD * ES + c * 16), sc);
      sc = valid ? sc * p.scale_log2 : -INFINITY;
      const float mn = fmaxf(m[hh], wave_max(sc));  // finite: every tile holds a live key
      const float alpha = fast_exp2(m[hh] - mn);
      const float pj = fast_exp2(sc - mn);
      m[hh] = mn;
      lsum[hh] = fmaf(lsum[hh], alpha, pj);
      o0[hh] *= alpha;
      o1[hh] *= alpha;
      // key j's probability goes where the lanes of sub-group j % KPS read it in order
      pb[wave][(lane % KPS) * RUN + lane / KPS] = pj;
      __builtin_amdgcn_wave_barrier();
      const float* pw = &pb[wave][sub * RUN];
#pragma unroll 2
      for (int i = 0; i < RUN; i += 4) {
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(pw + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const char* row = vs + ((i + e) * KPS + sub) * ROWB;
          float v0, v1;
          if (CDT == DT_F32) {
            const f32x2 vv = *reinterpret_cast<const f32x2*>(row + d0 * 4);
            v0 = vv[0];
            v1 = vv[1];
          } else {
            const uint32_t vv = *reinterpret_cast<const uint32_t*>(row + d0 * 2);
            const uint16_t lo = static_cast<uint16_t>(vv & 0xFFFF), hi = static_cast<uint16_t>(vv >> 16);
            v0 = CDT == DT_BF16 ? bf2f(lo) : h2f(lo);
            v1 = CDT == DT_BF16 ? bf2f(hi) : h2f(hi);
          }
          o0[hh] = fmaf(p4[e], v0, o0[hh]);
          o1[hh] = fmaf(p4[e], v1, o1[hh]);
        }
      }
      __builtin_amdgcn_wave_barrier();  // the next head rewrites pb only after these reads
    }
    __syncthreads();  // the tile's LDS rows are rewritten next iteration
  }

#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    if (hh >= nhw) break;
    float a = o0[hh], b = o1[hh];
    if (KPS == 2) {
      a += __shfl_xor(a, 32);
      b += __shfl_xor(b, 32);
    }
    const float l = wave_sum(lsum[hh]);
    const int64_t slot = (static_cast<int64_t>(g) * G + wave + 4 * hh) * p.nsplit + split;
    if (lane < LPK) *reinterpret_cast<f32x2*>(p.part_o + slot * HD + d0) = f32x2{a, b};
    if (lane == 0) *reinterpret_cast<f32x2*>(p.part_ml + slot * 2) = f32x2{m[hh], l};
  }
}

// out[h, d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s, M = max_s m_s; one workgroup
// per query head: the split weights are formed once in LDS, then thread d sums its column.
constexpr int kDecMaxSplits = 512;

__device__ __forceinline__ float block128_reduce(float v, bool is_max, float* red) {
  v = is_max ? wave_max(v) : wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = is_max ? fmaxf(red[0], red[1]) : red[0] + red[1];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(128) void decode_attn_combine_kernel(const float* part_o, const float* part_ml,
                                                                  int nsplit, int hd, float* out) {
  __shared__ float wsh[kDecMaxSplits];
  __shared__ float red[2];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float* ml = part_ml + static_cast<int64_t>(h) * nsplit * 2;
  float mx = -INFINITY;
  for (int s = tid; s < nsplit; s += 128) mx = fmaxf(mx, ml[2 * s]);
  mx = block128_reduce(mx, true, red);
  float l = 0.f;
  for (int s = tid; s < nsplit; s += 128) {
    const float w = fast_exp2(ml[2 * s] - mx);
    wsh[s] = w;
    l = fmaf(w, ml[2 * s + 1], l);
  }
  l = block128_reduce(l, false, red);   // its barriers also publish wsh
  if (tid >= hd) return;
  const float* po = part_o + static_cast<int64_t>(h) * nsplit * hd + tid;
  float acc = 0.f;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) acc = fmaf(wsh[s], po[static_cast<int64_t>(s) * hd], acc);
  out[static_cast<int64_t>(h) * hd + tid] = acc / l;
}

template <int CDT>
static hipError_t decode_partial_hd(const DecodeAttnParams& p, int hd, dim3 grid, hipStream_t s) {
  if (hd == 128) decode_attn_partial_kernel<CDT, 128><<<grid, 256, 0, s>>>(p);
  else if (hd == 64) decode_attn_partial_kernel<CDT, 64><<<grid, 256, 0, s>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_attention(const DecodeAttnParams& p, int hd, int cache_dt, float* out, hipStream_t s) {
  if (p.len < 1 || p.nkv < 1 || p.nh % p.nkv != 0 || p.nh / p.nkv > kDecMaxGroup) return hipErrorInvalidValue;
  if (p.nsplit != decode_num_splits(p.len, p.nkv) || p.tiles_per_split != decode_tiles_per_split(p.len, p.nkv) ||
      p.nsplit > kDecMaxSplits || hd > 128)
    return hipErrorInvalidValue;
  const dim3 grid(p.nsplit, p.nkv);
  hipError_t e;
  if (cache_dt == DT_F16) e = decode_partial_hd<DT_F16>(p, hd, grid, s);
  else if (cache_dt == DT_BF16) e = decode_partial_hd<DT_BF16>(p, hd, grid, s);
  else if (cache_dt == DT_F32) e = decode_partial_hd<DT_F32>(p, hd, grid, s);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  decode_attn_combine_kernel<<<p.nh, 128, 0, s>>>(p.part_o, p.part_ml, p.nsplit, hd, out);
  return hipGetLastError();
}

// ---- decode projections ---------------------------------------------------------------------
// Workgroup = 4 output rows (SwiGLU: 4 gate rows and the matching 4 up rows), its four waves
// splitting K; fp32 accumulation, wave reductions, then the four partial sums meet in LDS. The
// weight loads of U chunks of every row are issued together before any arithmetic (8 loads of
// 16 bytes in flight per wave), and even the smaller matrices spread over enough workgroups to
// hide the load latency.
constexpr int kGvRows = 4;

// 8 consecutive weights as raw 16-byte words (two words for fp32).
template <int DT>
struct Raw8 {
  u32x4 w[DT == DT_F32 ? 2 : 1];
};

template <int DT>
__device__ __forceinline__ Raw8<DT> load_raw8(const char* row, int i) {
  Raw8<DT> r;
  constexpr int ES = DT == DT_F32 ? 4 : 2;
#pragma unroll
  for (int h = 0; h < (DT == DT_F32 ? 2 : 1); ++h)
    r.w[h] = *reinterpret_cast<const u32x4*>(row + static_cast<int64_t>(i) * ES + 16 * h);
  return r;
}

template <int DT>
__device__ __forceinline__ float dot_raw8(const Raw8<DT>& r, const float (&x)[8], float acc) {
  if (DT == DT_F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t word = r.w[e >> 2][e & 3];
      acc = fmaf(__uint_as_float(word), x[e], acc);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t word = r.w[0][e];
      const uint16_t lo = static_cast<uint16_t>(word & 0xFFFF), hi = static_cast<uint16_t>(word >> 16);
      acc = fmaf(DT == DT_BF16 ? bf2f(lo) : h2f(lo), x[2 * e], acc);
      acc = fmaf(DT == DT_BF16 ? bf2f(hi) : h2f(hi), x[2 * e + 1], acc);
    }
  }
  return acc;
}

template <int DT, int EPI>
__global__ __launch_bounds__(256) void gemv_epi_kernel(GemvParams p) {
  constexpr int ES = DT == DT_F32 ? 4 : 2;
  constexpr int NR = EPI == GV_SWIGLU ? 2 * kGvRows : kGvRows;
  constexpr int U = (DT == DT_F32 ? 8 : 8) / NR > 0 ? (DT == DT_F32 ? 8 : 8) / NR : 1;  // chunks per row per pass
  __shared__ float red[4][NR];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // the workgroup's four waves share the same rows and split K: wave w takes the 8-element
  // chunks w*64 + lane, (w + 4)*64 + lane, ...
  const int r0 = blockIdx.x * kGvRows;
  // byte offset of row rr: row-major rr * K, or tiled (16-row groups of 32-column tiles): the
  // group's base plus 32 elements per row inside it; element i of a row then sits at i
  // (row-major) or (i / 32) * 512 + i % 32 (tiled) from there
  auto row_off = [&](int rr) -> int64_t {
    return (p.w_tiled ? static_cast<int64_t>(rr >> 4) * 16 * p.K + (rr & 15) * 32 : static_cast<int64_t>(rr) * p.K) * ES;
  };
  const char* rowp[NR];
#pragma unroll
  for (int j = 0; j < kGvRows; ++j) {
    const int r = min(r0 + j, p.rows - 1);  // rows past the end repeat the last (never stored)
    if (EPI == GV_SWIGLU) {
      rowp[j] = static_cast<const char*>(p.W0) + row_off(r);
      rowp[kGvRows + j] = static_cast<const char*>(p.W1) + row_off(r);
    } else {
      const void* W = r < p.nseg0 ? p.W0 : r < p.nseg1 ? p.W1 : p.W2;
      const int rr = r < p.nseg0 ? r : r < p.nseg1 ? r - p.nseg0 : r - p.nseg1;
      rowp[j] = static_cast<const char*>(W) + row_off(rr);
    }
  }
  float acc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = 0.f;
  // folded RMSNorm: the product runs on x * norm_w; sum of x^2 alongside, the row scale
  // 1/sqrt(mean + eps) applied to the finished dot products
  const bool nrm = p.norm_w != nullptr;
  float ss = 0.f;
  constexpr int STEP = 4 * 64 * 8;   // elements per pass of the four waves
  for (int i0 = (wave * 64 + lane) * 8; i0 < p.K; i0 += STEP * U) {
    Raw8<DT> w[U][NR];
    float xv[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(i0 + u * STEP, p.K - 8);   // chunks past the end repeat the last, weighted 0
      const int wi = p.w_tiled ? ((i >> 5) << 9) + (i & 31) : i;
#pragma unroll
      for (int j = 0; j < NR; ++j) w[u][j] = load_raw8<DT>(rowp[j], wi);
      load8<DT_F32>(p.x, i, xv[u]);
      if (i0 + u * STEP >= p.K) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[u][e] = 0.f;
      }
      if (nrm) {
        float gv[8];
        if (p.norm_dt == DT_BF16) load8<DT_BF16>(p.norm_w, i, gv);
        else if (p.norm_dt == DT_F16) load8<DT_F16>(p.norm_w, i, gv);
        else load8<DT_F32>(p.norm_w, i, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ss = fmaf(xv[u][e], xv[u][e], ss);
          xv[u][e] *= gv[e];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = dot_raw8<DT>(w[u][j], xv[u], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = wave_sum(acc[j]);
  __shared__ float red_ss[4];
  if (nrm) ss = wave_sum(ss);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < NR; ++j) red[wave][j] = acc[j];
    red_ss[wave] = ss;
  }
  __syncthreads();
  if (wave == 0 && lane < kGvRows && r0 + lane < p.rows) {
    float tot[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) tot[j] = (red[0][j] + red[1][j]) + (red[2][j] + red[3][j]);
    if (nrm) {
      const float sum_sq = (red_ss[0] + red_ss[1]) + (red_ss[2] + red_ss[3]);
      const float r = 1.0f / sqrtf(sum_sq / static_cast<float>(p.K) + p.eps);
#pragma unroll
      for (int j = 0; j < NR; ++j) tot[j] *= r;
    }
    float v = tot[0];
#pragma unroll
    for (int j = 1; j < kGvRows; ++j) v = lane == j ? tot[j] : v;
    const int r = r0 + lane;
    if (EPI == GV_SWIGLU) {
      float u = tot[kGvRows];
#pragma unroll
      for (int j = 1; j < kGvRows; ++j) u = lane == j ? tot[kGvRows + j] : u;
      v = v / (1.f + __expf(-v)) * u;
    } else if (EPI == GV_RESID) {
      v += p.R[r];
    }
    p.y[r] = v;
  }
}

template <int EPI>
static hipError_t gemv_dt(const GemvParams& p, int dt, unsigned blocks, hipStream_t s) {
  if (dt == DT_BF16) gemv_epi_kernel<DT_BF16, EPI><<<blocks, 256, 0, s>>>(p);
  else if (dt == DT_F16) gemv_epi_kernel<DT_F16, EPI><<<blocks, 256, 0, s>>>(p);
  else if (dt == DT_F32) gemv_epi_kernel<DT_F32, EPI><<<blocks, 256, 0, s>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvParams& p, int epi, int wdt, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  if (p.K % 8 != 0 || p.K <= 0) return hipErrorInvalidValue;
  // tiled weights: 16-bit, K a multiple of 32, every segment a whole number of row groups
  if (p.w_tiled && (wdt == DT_F32 || p.K % 32 != 0 || p.nseg0 % 16 != 0 || p.nseg1 % 16 != 0 || p.rows % 16 != 0))
    return hipErrorInvalidValue;
  const unsigned blocks = static_cast<unsigned>((p.rows + kGvRows - 1) / kGvRows);
  if (epi == GV_STORE) return gemv_dt<GV_STORE>(p, wdt, blocks, s);
  if (epi == GV_RESID) return gemv_dt<GV_RESID>(p, wdt, blocks, s);
  if (epi == GV_SWIGLU) return gemv_dt<GV_SWIGLU>(p, wdt, blocks, s);
  return hipErrorInvalidValue;
}

}  // namespace q3
