// Streaming (HBM-bound) kernels: row RMSNorm, the fused per-head q/k RMSNorm + interleaved
// MRoPE rotation, and the DeepStack row add.
//
// RMSNorm: cortiq-engine 0.8.21, qwen3te.rs, `rms_norm_into` (mean of squares, eps inside the
// square root, plain weight). q/k norm + rotation: the same page, `norm_rope` (norm before the
// rotation; split-half pairs (i, i + hd/2); Qwen3-VL's interleaved axis choice per pair).
// DeepStack: hf2q 0.1.1, qwen3vl_text/forward.rs, Phase D (add on image-token rows only).
#include "common.h"
#include "kernels.h"

#include <cmath>
#include <type_traits>

namespace q3 {

// ------------------------------------------------------------------------------------------
// RMSNorm: 256-thread workgroups, one row at a time; a row stays in registers between the
// sum-of-squares pass and the scaling pass, so x is read from HBM once.
constexpr int kNormThreads = 256;
constexpr int kNormGrid = 1024;  // workgroups of the streaming RMSNorm (4 per CU)
constexpr int kNormMaxVec = 16;  // float4 per thread: hidden <= 16384

// Load 4 consecutive elements (index 4c .. 4c+3) of a vector stored as dtype DT, as floats.
template <int DT>
__device__ __forceinline__ f32x4 load4(const void* p, int c) {
  if (DT == DT_F32) return reinterpret_cast<const f32x4*>(p)[c];
  const uint2 w = reinterpret_cast<const uint2*>(p)[c];
  if (DT == DT_BF16)
    return f32x4{bf2f(w.x & 0xFFFF), bf2f(w.x >> 16), bf2f(w.y & 0xFFFF), bf2f(w.y >> 16)};
  return f32x4{h2f(w.x & 0xFFFF), h2f(w.x >> 16), h2f(w.y & 0xFFFF), h2f(w.y >> 16)};
}

template <int DT>
__device__ __forceinline__ void store4(void* p, int64_t c, f32x4 v) {
  if (DT == DT_F32) {
    reinterpret_cast<f32x4*>(p)[c] = v;
  } else {
    uint2 o;
    o.x = DT == DT_BF16 ? pack2bf(v[0], v[1]) : Fmt<OP_F16>::pack2(v[0], v[1]);
    o.y = DT == DT_BF16 ? pack2bf(v[2], v[3]) : Fmt<OP_F16>::pack2(v[2], v[3]);
    reinterpret_cast<uint2*>(p)[c] = o;
  }
}

// Streaming form: a fixed grid of workgroups walks the rows (row r, r + grid, ...), loading the
// next row into registers while the current one is reduced and written, so reads and writes
// overlap instead of alternating in bursts. NV float4 per thread per row; FULL: hidden is
// exactly 4 * NV * kNormThreads, so no chunk needs a bounds check and every load is issued
// unconditionally.
template <int W_DT, int Y_DT, int NV, bool FULL>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_stream_kernel(const float* __restrict__ x,
                                                                      const void* __restrict__ w,
                                                                      void* __restrict__ y, int rows,
                                                                      int hidden, float eps, int tiled) {
  const int nv = hidden >> 2;
  // output index of float4 c of a row (4-element units): row-major row * nv + c; tiled (16-bit
  // y): the row's base inside its 16-row group plus 128 per 32 columns
  const int c_ks = tiled ? 128 : 8;
  f32x4 g[NV], cur[NV], nxt[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * kNormThreads;
    if (FULL || c < nv) g[i] = load4<W_DT>(w, c);
  }
  auto load_row = [&](f32x4 (&v)[NV], int row) {
    const f32x4* xr = reinterpret_cast<const f32x4*>(x + static_cast<int64_t>(row) * hidden);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = threadIdx.x + i * kNormThreads;
      if (FULL || c < nv) v[i] = xr[c];
    }
  };
  __shared__ float red[2][kNormThreads / 64];
  // the grid never exceeds the rows, so every workgroup has a first row; past its last row a
  // workgroup loads its current row again (cached, never used)
  int row = blockIdx.x;
  load_row(cur, row);
  for (int it = 0; row < rows; row += gridDim.x, ++it) {
    const int rn = row + gridDim.x;
    load_row(nxt, rn < rows ? rn : row);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = threadIdx.x + i * kNormThreads;
      if (FULL || c < nv) ss += cur[i][0] * cur[i][0] + cur[i][1] * cur[i][1] + cur[i][2] * cur[i][2] + cur[i][3] * cur[i][3];
    }
    ss = wave_sum(ss);
    // two reduction slots by row parity: a slot is rewritten two rows later, after every thread
    // has passed the barrier of the row in between
    if ((threadIdx.x & 63) == 0) red[it & 1][threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kNormThreads / 64; ++i) tot += red[it & 1][i];
    const float r = 1.0f / sqrtf(tot / static_cast<float>(hidden) + eps);
    const int64_t y_row = tiled ? static_cast<int64_t>(row >> 4) * 4 * hidden + (row & 15) * 8
                                : static_cast<int64_t>(row) * nv;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = threadIdx.x + i * kNormThreads;
      if (FULL || c < nv) {
        const f32x4 o = {cur[i][0] * r * g[i][0], cur[i][1] * r * g[i][1], cur[i][2] * r * g[i][2],
                         cur[i][3] * r * g[i][3]};
        store4<Y_DT>(y, y_row + (c >> 3) * c_ks + (c & 7), o);
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) cur[i] = nxt[i];
  }
}

template <int W_DT, int Y_DT>
static void rms_launch_k(const float* x, const void* w, void* y, int rows, int hidden, float eps,
                         int tiled, hipStream_t s) {
  const int grid = rows < kNormGrid ? rows : kNormGrid;
  auto go = [&](auto nv) {
    constexpr int NV = decltype(nv)::value;
    if (hidden == 4 * kNormThreads * NV)
      rmsnorm_stream_kernel<W_DT, Y_DT, NV, true><<<grid, kNormThreads, 0, s>>>(x, w, y, rows, hidden, eps, tiled);
    else
      rmsnorm_stream_kernel<W_DT, Y_DT, NV, false><<<grid, kNormThreads, 0, s>>>(x, w, y, rows, hidden, eps, tiled);
  };
  if (hidden <= 4 * kNormThreads * 4) go(std::integral_constant<int, 4>{});
  else if (hidden <= 4 * kNormThreads * 8) go(std::integral_constant<int, 8>{});
  else go(std::integral_constant<int, 16>{});
}

template <int W_DT>
static hipError_t rms_launch_y(const float* x, const void* w, void* y, int y_dt, int rows, int hidden,
                               float eps, int tiled, hipStream_t s) {
  switch (y_dt) {
    case DT_F32: rms_launch_k<W_DT, DT_F32>(x, w, y, rows, hidden, eps, 0, s); break;
    case DT_BF16: rms_launch_k<W_DT, DT_BF16>(x, w, y, rows, hidden, eps, tiled, s); break;
    case DT_F16: rms_launch_k<W_DT, DT_F16>(x, w, y, rows, hidden, eps, tiled, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, const void* w, int w_dt, void* y, int y_dt, int rows,
                          int hidden, float eps, hipStream_t s, bool y_tiled) {
  if (rows <= 0) return hipSuccess;
  if (hidden % 4 != 0 || hidden > 4 * kNormThreads * kNormMaxVec) return hipErrorInvalidValue;
  if (y_tiled && (y_dt == DT_F32 || hidden % 32 != 0)) return hipErrorInvalidValue;
  const int t = y_tiled ? 1 : 0;
  switch (w_dt) {
    case DT_F32: return rms_launch_y<DT_F32>(x, w, y, y_dt, rows, hidden, eps, t, s);
    case DT_BF16: return rms_launch_y<DT_BF16>(x, w, y, y_dt, rows, hidden, eps, t, s);
    case DT_F16: return rms_launch_y<DT_F16>(x, w, y, y_dt, rows, hidden, eps, t, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------------------------------
// DeepStack: one workgroup per slab row. The row list was checked on the host (strictly
// increasing, inside [0, S)), so no two workgroups touch the same output row.
__device__ __forceinline__ float load_elem(const void* p, int64_t i, int dt) {
  if (dt == DT_F32) return static_cast<const float*>(p)[i];
  const uint16_t h = static_cast<const uint16_t*>(p)[i];
  return dt == DT_BF16 ? bf2f(h) : h2f(h);
}

__global__ __launch_bounds__(256) void deepstack_add_kernel(float* __restrict__ y,
                                                            const int32_t* __restrict__ rows,
                                                            const void* __restrict__ ds, int ds_dt,
                                                            int S, int hidden) {
  const int i = blockIdx.x;
  const int r = rows[i];
  if (r < 0 || r >= S) return;  // never taken for a checked list; keeps the store in bounds
  float* yr = y + static_cast<int64_t>(r) * hidden;
  for (int c = threadIdx.x; c < hidden; c += 256) {
    yr[c] += load_elem(ds, static_cast<int64_t>(i) * hidden + c, ds_dt);
  }
}

hipError_t launch_deepstack_add(float* y, const int32_t* rows, const void* ds, int ds_dt, int n,
                                int S, int hidden, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  deepstack_add_kernel<<<n, 256, 0, s>>>(y, rows, ds, ds_dt, S, hidden);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// q/k RMSNorm + interleaved MRoPE. One 256-thread workgroup per four tokens. A lane owns eight
// consecutive rotation pairs (x_i, x_{i+hd/2}), i = i0 .. i0+7, of one head row, read and written
// with 16-byte accesses (two for fp32), so the rotation is lane-local and the hd/16 lanes of a row
// reduce the sum of squares with cross-lane shuffles. The angle of pair i
// depends on the token only (not the head): the workgroup forms each of its tokens' hd/2
// cos/sin pairs once, in LDS, and every lane applies its four to each q and k head row it owns;
// the norm weights are read once per lane.
//
// Angle precision: theta^(-2i/hd) is formed in double on the host, phi = pos * theta^(-2i/hd)
// in double and reduced to [-pi, pi] in double before the single-precision sincos, so its
// error does not grow with the position.
// tokens per workgroup: the norm weights and the workgroup set-up are shared by this many
// tokens (four: 32 -> 24 us for the 8B q/k at 4096 tokens, against one token per workgroup)
constexpr int kRopeTokens = 4;
// rotation pairs per lane: 8 (16-byte accesses for 16-bit rows; 6% faster than 4 at the 8B shape)
constexpr int kRopePairs = 8;
// below this many token blocks (fewer than the CUs) the launch splits each token's head rows
// over workgroups instead
constexpr int kRopeSplitBelow = 256;
struct RopeFreqs {
  double inv[64];
};

template <int DT>
__device__ __forceinline__ void load4(const void* row, int i, float (&v)[4]) {
  if (DT == DT_F32) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = w[e];
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(row) + i);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint16_t lo = static_cast<uint16_t>(w[e] & 0xFFFF), hi = static_cast<uint16_t>(w[e] >> 16);
      v[2 * e] = DT == DT_BF16 ? bf2f(lo) : h2f(lo);
      v[2 * e + 1] = DT == DT_BF16 ? bf2f(hi) : h2f(hi);
    }
  }
}

template <int DT>
__device__ __forceinline__ void store4(void* row, int i, const float (&v)[4]) {
  if (DT == DT_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(row) + i) = f32x4{v[0], v[1], v[2], v[3]};
  } else {
    u32x2 w;
#pragma unroll
    for (int e = 0; e < 2; ++e)
      w[e] = DT == DT_BF16 ? Fmt<OP_BF16>::pack2(v[2 * e], v[2 * e + 1]) : Fmt<OP_F16>::pack2(v[2 * e], v[2 * e + 1]);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(row) + i) = w;
  }
}

// PPL consecutive elements (4 or 8) of a row at element i, as floats, and back
template <int DT, int PPL>
__device__ __forceinline__ void ld_run(const void* row, int i, float (&v)[PPL]) {
  if constexpr (PPL == 4) load4<DT>(row, i, v);
  else load8<DT>(row, i, v);
}
template <int DT, int PPL>
__device__ __forceinline__ void st_run(void* row, int i, const float (&v)[PPL]) {
  if constexpr (PPL == 4) store4<DT>(row, i, v);
  else store8<DT>(row, i, v);
}
// the same store for a row of runtime type dt (cache rows)
template <int PPL>
__device__ __forceinline__ void st_run_dt(void* row, int i, const float (&v)[PPL], int dt) {
  if (dt == DT_F32) st_run<DT_F32, PPL>(row, i, v);
  else if (dt == DT_BF16) st_run<DT_BF16, PPL>(row, i, v);
  else st_run<DT_F16, PPL>(row, i, v);
}

template <int DT, int HD, int TPW, int PPL>
__global__ __launch_bounds__(256) void qk_norm_mrope_kernel(const RopeParams p, const RopeFreqs f) {
  const double* inv_freq = f.inv;
  constexpr int HALF = HD / 2;
  constexpr int LPR = HALF / PPL;                   // lanes per head row
  constexpr int ROWS_PER_WAVE = 64 / LPR;
  constexpr int ROWS_PER_PASS = 4 * ROWS_PER_WAVE;  // 4 waves
  static_assert(TPW * HALF <= 256, "one angle per thread");
  const int s0 = blockIdx.x * TPW;
  const int lane = threadIdx.x & 63;
  const int i0 = PPL * (lane % LPR);
  const int sub = (threadIdx.x >> 6) * ROWS_PER_WAVE + lane / LPR;

  // head rows of the TPW tokens in token order: row index hh = token * (nh + nkv) + head.
  // With gridDim.y > 1 the q/k workgroups of a token block take every qk_groups-th pass of
  // rows, and with a cache to fill the last workgroup appends the v rows alone.
  const int nrows = p.nh + p.nkv;
  const int gy = static_cast<int>(gridDim.y), by = static_cast<int>(blockIdx.y);
  const int qk_groups = (p.kc && gy > 1) ? gy - 1 : gy;
  const int stride = ROWS_PER_PASS * qk_groups;
  auto valid_row = [&](int hh) { return hh < TPW * nrows && s0 + (TPW == 1 ? 0 : hh / nrows) < p.S; };
  auto row_at = [&](int hh, int& tt, int& h) -> void* {
    tt = TPW == 1 ? 0 : hh / nrows;
    h = TPW == 1 ? hh : hh - tt * nrows;
    const int64_t s = s0 + tt;
    return h < p.nh ? static_cast<void*>(static_cast<char*>(p.q) +
                                         (s * p.q_stride + static_cast<int64_t>(h) * HD) * (DT == DT_F32 ? 4 : 2))
                    : static_cast<void*>(static_cast<char*>(p.k) +
                                         (s * p.k_stride + static_cast<int64_t>(h - p.nh) * HD) * (DT == DT_F32 ? 4 : 2));
  };
  // the first row's loads and the lane's norm weights (entries i0.. and i0+hd/2.. of each,
  // one vector load per run, the dtype resolved once) go out before the angles are formed
  int hh = by < qk_groups ? sub + by * ROWS_PER_PASS : TPW * nrows;
  bool ok = valid_row(hh);
  int tt = 0, h = 0;
  // (a lane group without rows loads row 0 of token s0, which every launched workgroup has,
  // and never uses it: the loads stay unconditional)
  void* row = row_at(ok ? hh : 0, tt, h);
  float a[PPL], b[PPL];
  ld_run<DT, PPL>(row, i0, a);
  ld_run<DT, PPL>(row, i0 + HALF, b);
  float qa[PPL], qb[PPL], ka[PPL], kb[PPL];
  auto load_norms = [&](auto dt) {
    constexpr int ND = decltype(dt)::value;
    ld_run<ND, PPL>(p.q_norm, i0, qa);
    ld_run<ND, PPL>(p.q_norm, i0 + HALF, qb);
    ld_run<ND, PPL>(p.k_norm, i0, ka);
    ld_run<ND, PPL>(p.k_norm, i0 + HALF, kb);
  };
  if (p.norm_dt == DT_BF16) load_norms(std::integral_constant<int, DT_BF16>{});
  else if (p.norm_dt == DT_F16) load_norms(std::integral_constant<int, DT_F16>{});
  else load_norms(std::integral_constant<int, DT_F32>{});

  // the hd/2 angles of each of the workgroup's TPW tokens, each formed once (thread
  // t*hd/2 + i forms angle i of token s0 + t) and shared through LDS
  __shared__ __attribute__((aligned(16))) float s_cs[TPW][HALF];
  __shared__ __attribute__((aligned(16))) float s_sn[TPW][HALF];
  if (threadIdx.x < TPW * HALF) {
    const int ta = threadIdx.x / HALF;
    const int i = threadIdx.x % HALF;
    const int s = s0 + ta;
    if (s < p.S) {
      int axis = 0;
      if (i % 3 == 1 && i < 3 * p.sec_h) axis = 1;
      else if (i % 3 == 2 && i < 3 * p.sec_w) axis = 2;
      const double pos = static_cast<double>(p.pos[static_cast<int64_t>(axis) * p.S + s]);
      const double phi = pos * inv_freq[i];
      const double two_pi = 6.283185307179586476925286766559;
      const double red = fma(-two_pi, rint(phi * (1.0 / two_pi)), phi);
      sincosf(static_cast<float>(red), &s_sn[ta][i], &s_cs[ta][i]);
    }
  }
  __syncthreads();

  // Each row's successor (same lane group, the next pass) is loaded before the row is
  // written back, so its load overlaps this row's arithmetic and stores; past the last row the
  // current row is loaded again and never used.
  while (ok) {
    const int hn = hh + stride;
    const bool okn = valid_row(hn);
    int ttn = tt, hnh = h;
    void* rown = okn ? row_at(hn, ttn, hnh) : row;
    float na[PPL], nb[PPL];
    ld_run<DT, PPL>(rown, i0, na);
    ld_run<DT, PPL>(rown, i0 + HALF, nb);
    const int s = s0 + tt;
    const bool is_q = h < p.nh;
    float cs[PPL], sn[PPL];
#pragma unroll
    for (int e4 = 0; e4 < PPL; e4 += 4) {
      const f32x4 c4 = *reinterpret_cast<const f32x4*>(&s_cs[tt][i0 + e4]);
      const f32x4 n4 = *reinterpret_cast<const f32x4*>(&s_sn[tt][i0 + e4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cs[e4 + e] = c4[e];
        sn[e4 + e] = n4[e];
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < PPL; ++e) ss = fmaf(a[e], a[e], fmaf(b[e], b[e], ss));
    ss = group_sum(ss, LPR);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(HD) + p.eps);
    float ra[PPL], rb[PPL];
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
      const float x = a[e] * r * (is_q ? qa[e] : ka[e]);
      const float y = b[e] * r * (is_q ? qb[e] : kb[e]);
      ra[e] = x * cs[e] - y * sn[e];
      rb[e] = x * sn[e] + y * cs[e];
    }
    st_run<DT, PPL>(row, i0, ra);
    st_run<DT, PPL>(row, i0 + HALF, rb);
    if (p.kc && !is_q) {
      const int es = p.cache_dt == DT_F32 ? 4 : 2;
      void* crow = static_cast<char*>(p.kc) +
                   ((static_cast<int64_t>(h - p.nh) * p.capacity + p.row0 + s) * HD) * es;
      st_run_dt<PPL>(crow, i0, ra, p.cache_dt);
      st_run_dt<PPL>(crow, i0 + HALF, rb, p.cache_dt);
    }
    hh = hn;
    ok = okn;
    tt = ttn;
    h = hnh;
    row = rown;
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
      a[e] = na[e];
      b[e] = nb[e];
    }
  }
  // cache append of the tokens' v rows (same lane layout, no arithmetic)
  if (p.kc && (gy == 1 || by == gy - 1)) {
    for (int hv = sub; hv < TPW * p.nkv; hv += ROWS_PER_PASS) {
      const int tv = TPW == 1 ? 0 : hv / p.nkv;
      const int g = hv - tv * p.nkv;
      const int s = s0 + tv;
      if (s >= p.S) break;
      const void* vrow = static_cast<const char*>(p.v) +
                         (static_cast<int64_t>(s) * p.v_stride + static_cast<int64_t>(g) * HD) * (DT == DT_F32 ? 4 : 2);
      float a[PPL], b[PPL];
      ld_run<DT, PPL>(vrow, i0, a);
      ld_run<DT, PPL>(vrow, i0 + HALF, b);
      const int es = p.cache_dt == DT_F32 ? 4 : 2;
      void* crow = static_cast<char*>(p.vc) + ((static_cast<int64_t>(g) * p.capacity + p.row0 + s) * HD) * es;
      st_run_dt<PPL>(crow, i0, a, p.cache_dt);
      st_run_dt<PPL>(crow, i0 + HALF, b, p.cache_dt);
    }
  }
}

template <int HD, int TPW>
static hipError_t rope_launch_t(const RopeParams& p, int dt, dim3 grid, const RopeFreqs& f, hipStream_t s) {
  const dim3 block(256);
  switch (dt) {
    case DT_F32: qk_norm_mrope_kernel<DT_F32, HD, TPW, kRopePairs><<<grid, block, 0, s>>>(p, f); break;
    case DT_BF16: qk_norm_mrope_kernel<DT_BF16, HD, TPW, kRopePairs><<<grid, block, 0, s>>>(p, f); break;
    case DT_F16: qk_norm_mrope_kernel<DT_F16, HD, TPW, kRopePairs><<<grid, block, 0, s>>>(p, f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int HD>
static hipError_t rope_launch(const RopeParams& p, int dt, hipStream_t s) {
  // theta^(-2i/hd) for i < hd/2, in double on the host, passed with the launch
  RopeFreqs f;
  for (int i = 0; i < HD / 2; ++i) f.inv[i] = std::exp2(-(2.0 * i / HD) * p.log2_theta);
  constexpr int TPW = kRopeTokens;
  const int blocks = (p.S + TPW - 1) / TPW;
  if (blocks >= kRopeSplitBelow) return rope_launch_t<HD, TPW>(p, dt, dim3(blocks), f, s);
  // few tokens (decode, short prompts): one token per workgroup and its head rows split over
  // workgroups, one pass of rows each, so that no workgroup runs passes one after another
  constexpr int LPR = HD / 2 / kRopePairs;
  constexpr int ROWS_PER_PASS = 4 * (64 / LPR);
  const int passes = (p.nh + p.nkv + ROWS_PER_PASS - 1) / ROWS_PER_PASS;
  return rope_launch_t<HD, 1>(p, dt, dim3(p.S, passes + (p.kc ? 1 : 0)), f, s);
}

hipError_t launch_qk_norm_mrope(const RopeParams& p, int head_dim, int data_dt, hipStream_t s) {
  if (p.S <= 0) return hipSuccess;
  if (head_dim == 128) return rope_launch<128>(p, data_dt, s);
  if (head_dim == 64) return rope_launch<64>(p, data_dt, s);
  return hipErrorInvalidValue;
}

}  // namespace q3
