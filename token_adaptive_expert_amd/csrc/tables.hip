// Offline per-expert tables A^GSP and A^RCR built from a layer's own weights.
//
// Method: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
// (picx.dev summary page), Methodology section 1 (GSP: a^up = ‖ΓW^up‖_F ·
// ‖ΓW^gate W^down‖_F, a^gate = ‖ΓW^gate‖_F · ‖ΓW^up W^down‖_F, their geometric
// mean, normalised by the layer mean) and section 2 (RCR: centred router rows,
// RMS-normalised prototype q, amplification ‖f(q)‖ / ‖q‖, normalised the same
// way).  Page convention: W^gate, W^up are H×I (w_gate[e] transposed here),
// W^down is I×H (w_down[e] transposed), Γ = diag(γ).
//
// GSP never forms an H×H product.  With the I×I Gram matrices
//   G_g = (ΓW^gate)ᵀ(ΓW^gate),  G_u = (ΓW^up)ᵀ(ΓW^up),  D = W^down W^downᵀ,
// ‖ΓW^gate W^down‖²_F = ⟨G_g, D⟩, ‖ΓW^up W^down‖²_F = ⟨G_u, D⟩ and
// ‖ΓW‖²_F = trace(G).  Each Gram contracts over H along rows of an I×H
// matrix: w_gate[e] / w_up[e] rows as stored, and w_down[e] transposed once
// into the workspace.  G[i][j] = Σ_h w[i][h] · (γ_h² w[j][h]); for bf16 weights
// the second operand γ²w is split exactly into three bf16 planes while it is
// staged into LDS, so every MFMA product is exact and only the float32
// accumulation rounds.  The Gram kernel computes one 128×128 tile of the upper
// triangle of D, then G_g, then G_u, and folds ⟨G, D⟩ and the traces into
// per-tile float64 partials, so no Gram matrix is ever stored.
//
// RCR runs as three bandwidth-bound passes over the weights (prototype, then
// the gate/up rows, then the down rows) spread over many workgroups, and one
// final kernel reduces every per-expert partial in a fixed order.
#include "kernels.h"

#include <algorithm>

namespace ace {

namespace {

constexpr int GT = 128;         // Gram tile edge
constexpr int GPITCH = 80;      // LDS row pitch in bytes: 64-byte k-step + 16 padding
constexpr int GNW = 8;          // waves per Gram workgroup, each a 32x64 sub-tile
constexpr int GNTHR = GNW * 64;
constexpr int NXCD = 8;         // accelerator dies; workgroup i runs on die i % 8
constexpr int RROWS = 64;       // rows per RCR workgroup (16 per wave)
constexpr size_t WDT_CAP = size_t(512) << 20;  // bytes of transposed w_down per batch

template <typename T> struct GramPlanes;
template <> struct GramPlanes<bf16_t> { static constexpr int N = 3; };
template <> struct GramPlanes<float> { static constexpr int N = 1; };

// ---------------------------------------------------------------------------
// w_down[e] [H][I] -> wdT[b] [I][H] for experts e0 .. e0+nb-1 (64x64 LDS tiles).
// grid (I/64, H/64, nb), 256 threads.
template <typename T>
__global__ __launch_bounds__(256) void tables_transpose_kernel(TablesArgs a, int e0) {
  __shared__ T tile[64][65];
  const int ib = blockIdx.x, hb = blockIdx.y, b = blockIdx.z;
  const int H = a.H, I = a.I;
  const T* src = reinterpret_cast<const T*>(a.w_down) + (int64_t(e0) + b) * int64_t(H) * I;
  T* dst = reinterpret_cast<T*>(a.ws_wdT) + int64_t(b) * int64_t(I) * H;
  const int c = threadIdx.x & 63, r0 = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = r0 + 4 * j;  // h within the tile
    tile[r][c] = src[int64_t(hb * 64 + r) * I + ib * 64 + c];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = r0 + 4 * j;  // i within the tile
    dst[int64_t(ib * 64 + r) * H + hb * 64 + c] = tile[c][r];
  }
}

// One Gram unit of a 128x128 tile: acc = A-rows · op(B-rows)ᵀ over the whole
// H, where op is the identity (SPLIT false) or γ²-scaling followed by the
// exact plane split (SPLIT true).  ra / rb point at the first of the tile's
// 128 rows.  Wave w owns rows 32(w/2).. and cols 64(w%2).. of the tile;
// acc[x][y] is its 16x16 block (x, y) in the MFMA output layout.
template <typename T, bool SPLIT>
__device__ __forceinline__ void gram_unit(const T* __restrict__ ra, const T* __restrict__ rb,
                                          const float* __restrict__ gamma, int H, uint8_t* s_a, uint8_t* s_b,
                                          f32x4 (&acc)[2][4]) {
  constexpr int EPL = St<T>::EPL;
  constexpr int KS = 4 * EPL;                             // k values per 64-byte k-step
  constexpr int NP = SPLIT ? GramPlanes<T>::N : 1;
  constexpr int ABUF = GT * GPITCH;                       // bytes of one A buffer (= one plane)
  constexpr int BBUF = GramPlanes<T>::N * GT * GPITCH;    // bytes of one B buffer (all planes)
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int q = l >> 4, r16 = l & 15;
  const int wr = (w >> 1) * 32, wc = (w & 1) * 64;
  // this thread's staging unit: tile row r, 16-byte segment seg of the k-step
  const int r = tid >> 2, seg = tid & 3;
  const T* pa = ra + int64_t(r) * H + seg * EPL;
  const T* pb = rb + int64_t(r) * H + seg * EPL;
  const int so = r * GPITCH + seg * 16;
  const int nks = H / KS;

#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  float g[EPL];
  auto load_g = [&](int j) {
    if constexpr (SPLIT) {
      const float* gp = gamma + j * KS + seg * EPL;
#pragma unroll
      for (int u = 0; u < EPL / 4; ++u) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(gp + 4 * u);
#pragma unroll
        for (int v = 0; v < 4; ++v) g[4 * u + v] = t[v];
      }
    }
  };
  auto stage = [&](int buf, u32x4 va, u32x4 vb) {
    *reinterpret_cast<u32x4*>(s_a + buf * ABUF + so) = va;
    if constexpr (!SPLIT) {
      *reinterpret_cast<u32x4*>(s_b + buf * BBUF + so) = vb;
    } else if constexpr (GramPlanes<T>::N == 3) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[2 * u] = (g[2 * u] * g[2 * u]) * bf16_to_f32(uint16_t(vb[u] & 0xFFFFu));
        v[2 * u + 1] = (g[2 * u + 1] * g[2 * u + 1]) * bf16_to_f32(uint16_t(vb[u] >> 16));
      }
      u32x4 pl[3];
      split3_f8(v, pl);
#pragma unroll
      for (int p = 0; p < 3; ++p) *reinterpret_cast<u32x4*>(s_b + buf * BBUF + p * ABUF + so) = pl[p];
    } else {
      u32x4 o;
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = __float_as_uint((g[u] * g[u]) * __uint_as_float(vb[u]));
      *reinterpret_cast<u32x4*>(s_b + buf * BBUF + so) = o;
    }
  };

  u32x4 va = ld16(pa), vb = ld16(pb);
  load_g(0);
  stage(0, va, vb);
  __syncthreads();
  for (int j = 0; j < nks; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < nks;
    if (more) {
      va = ld16(pa + int64_t(j + 1) * KS);
      vb = ld16(pb + int64_t(j + 1) * KS);
      load_g(j + 1);
    }
    u32x4 fa[2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
      fa[x] = *reinterpret_cast<const u32x4*>(s_a + buf * ABUF + (wr + 16 * x + r16) * GPITCH + q * 16);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      u32x4 fb[4];
#pragma unroll
      for (int y = 0; y < 4; ++y)
        fb[y] = *reinterpret_cast<const u32x4*>(s_b + buf * BBUF + p * ABUF + (wc + 16 * y + r16) * GPITCH + q * 16);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = mma_step<T>(fa[x], fb[y], acc[x][y]);
    }
    if (more) stage(buf ^ 1, va, vb);
    __syncthreads();
  }
}

// grid: NXCD * ceil(nb * ntiles / NXCD) workgroups over the upper-triangular
// 128x128 tiles of every expert in the batch; consecutive tiles (those of one
// expert) run on one die, so its row blocks are reused from that die's L2.
template <typename T>
__global__ __launch_bounds__(GNTHR) void tables_gram_kernel(TablesArgs a, int e0, int nb) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2 * GT * GPITCH];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2 * GramPlanes<T>::N * GT * GPITCH];
  __shared__ double s_red[GNW][4];
  const int H = a.H, I = a.I;
  const int nbk = I / GT;
  const int ntiles = nbk * (nbk + 1) / 2;
  const int total = nb * ntiles;
  const int per = (total + NXCD - 1) / NXCD;
  const int g = int(blockIdx.x % NXCD) * per + int(blockIdx.x / NXCD);
  if (g >= total) return;
  const int b = g / ntiles;
  const int tile_id = g % ntiles;
  int t = tile_id, bi = 0;  // tile -> (bi, bj), bi <= bj, row-major over the upper triangle
  while (t >= nbk - bi) {
    t -= nbk - bi;
    ++bi;
  }
  const int bj = bi + t;
  const bool diag = bi == bj;
  const int64_t IH = int64_t(I) * H;
  const int64_t e = int64_t(e0) + b;
  const T* wdT = reinterpret_cast<const T*>(a.ws_wdT) + int64_t(b) * IH;
  const T* wg = reinterpret_cast<const T*>(a.w_gate) + e * IH;
  const T* wu = reinterpret_cast<const T*>(a.w_up) + e * IH;
  const int64_t oi = int64_t(bi) * GT * H, oj = int64_t(bj) * GT * H;

  f32x4 accd[2][4], acc[2][4];
  gram_unit<T, false>(wdT + oi, wdT + oj, a.gamma, H, s_a, s_b, accd);

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int q = l >> 4, r16 = l & 15;
  const int wr = (w >> 1) * 32, wc = (w & 1) * 64;
  double v[4];  // ⟨G_g,D⟩, ⟨G_u,D⟩, trace G_g, trace G_u over this tile
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const T* src = m == 0 ? wg : wu;
    gram_unit<T, true>(src + oi, src + oj, a.gamma, H, s_a, s_b, acc);
    double p = 0.0, tr = 0.0;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          p += double(acc[x][y][jj]) * double(accd[x][y][jj]);
          if (diag && wr + 16 * x + 4 * q + jj == wc + 16 * y + r16) tr += double(acc[x][y][jj]);
        }
    v[m] = p;
    v[2 + m] = tr;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    double x = v[c];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    v[c] = x;
  }
  if (l == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) s_red[w][c] = v[c];
  }
  __syncthreads();
  if (tid < 4) {
    double x = 0.0;
    for (int ww = 0; ww < GNW; ++ww) x += s_red[ww][tid];
    // an off-diagonal tile also stands for its mirror in the inner products
    if (tid < 2 && !diag) x *= 2.0;
    a.ws_part[(int64_t(b) * ntiles + tile_id) * 4 + tid] = x;
  }
}

// One thread per expert of the batch: sum its tile partials in tile order.
__global__ void tables_gsp_reduce_kernel(TablesArgs a, int e0, int nb) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  const int nbk = a.I / GT, ntiles = nbk * (nbk + 1) / 2;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int t = 0; t < ntiles; ++t)
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] += a.ws_part[(int64_t(b) * ntiles + t) * 4 + c];
  // s0 = ‖ΓW^gate W^down‖², s1 = ‖ΓW^up W^down‖², s2 = ‖ΓW^gate‖², s3 = ‖ΓW^up‖²
  const double a_up = sqrt(s[3]) * sqrt(s[0]);
  const double a_gate = sqrt(s[2]) * sqrt(s[1]);
  a.ws_raw_gsp[e0 + b] = sqrt(a_up * a_gate);
}

// ---------------------------------------------------------------------------
// RCR.  Mean router row over experts (float64 sums).
__global__ void tables_rcr_mean_kernel(TablesArgs a) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= a.H) return;
  double s = 0.0;
  for (int e = 0; e < a.E; ++e) s += a.w_router[int64_t(e) * a.H + h];
  a.ws_mean[h] = float(s / a.E);
}

__device__ __forceinline__ float block_sum256(float v, float* s_red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  return s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

// Prototype of expert e (one workgroup): q = w̃ / (RMS(w̃) + ε) with ρ = 1;
// stores x_e = q ⊙ γ (q in the role of x̄, so the expert sees x̄Γ) and ‖q‖.
__global__ __launch_bounds__(256) void tables_rcr_proto_kernel(TablesArgs a) {
  __shared__ float s_red[4];
  const int e = blockIdx.x, H = a.H;
  const float* wr = a.w_router + int64_t(e) * H;
  float* xe = a.ws_x + int64_t(e) * H;
  float ss = 0.f;
  for (int h = threadIdx.x; h < H; h += 256) {
    const float c = wr[h] - a.ws_mean[h];
    ss += c * c;
  }
  const float den = sqrtf(block_sum256(ss, s_red) / float(H)) + a.eps;
  float qq = 0.f;
  for (int h = threadIdx.x; h < H; h += 256) {
    const float qv = (wr[h] - a.ws_mean[h]) / den;
    qq += qv * qv;
    xe[h] = qv * a.gamma[h];
  }
  const float qn = sqrtf(block_sum256(qq, s_red));
  if (threadIdx.x == 0) a.ws_qnorm[e] = qn;
}

// Lane partial of the dot product of one weight row (len elements, read in
// 16-byte chunks) with a float32 vector; the caller reduces over the wave.
template <typename T>
__device__ __forceinline__ float row_dot(const T* row, const float* x, int len) {
  constexpr int EPL = St<T>::EPL;
  float s = 0.f;
  for (int c = lane_id(); c < len / EPL; c += 64) {
    const u32x4 v = ld16(row + c * EPL);
    const float* xp = x + c * EPL;
    if constexpr (EPL == 8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s += bf16_to_f32(uint16_t(v[u] & 0xFFFFu)) * xp[2 * u];
        s += bf16_to_f32(uint16_t(v[u] >> 16)) * xp[2 * u + 1];
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) s += __uint_as_float(v[u]) * xp[u];
    }
  }
  return s;
}

// v_e[i] = SiLU(w_gate[e][i] · x_e) · (w_up[e][i] · x_e); grid (I/RROWS, E).
template <typename T>
__global__ __launch_bounds__(256) void tables_rcr_up_kernel(TablesArgs a) {
  const int e = blockIdx.y, H = a.H, I = a.I;
  const float* xe = a.ws_x + int64_t(e) * H;
  const T* wg = reinterpret_cast<const T*>(a.w_gate) + int64_t(e) * I * H;
  const T* wu = reinterpret_cast<const T*>(a.w_up) + int64_t(e) * I * H;
  const int i0 = blockIdx.x * RROWS + wave_id() * (RROWS / 4);
  for (int i = i0; i < i0 + RROWS / 4; ++i) {
    const float g = wave_sum(row_dot<T>(wg + int64_t(i) * H, xe, H));
    const float u = wave_sum(row_dot<T>(wu + int64_t(i) * H, xe, H));
    if (lane_id() == 0) a.ws_v[int64_t(e) * I + i] = g / (1.0f + expf(-g)) * u;
  }
}

// Partial ‖f(q)‖² over RROWS output rows: Σ_h (w_down[e][h] · v_e)²; grid (H/RROWS, E).
template <typename T>
__global__ __launch_bounds__(256) void tables_rcr_down_kernel(TablesArgs a) {
  __shared__ float s_red[4];
  const int e = blockIdx.y, H = a.H, I = a.I;
  const float* ve = a.ws_v + int64_t(e) * I;
  const T* wd = reinterpret_cast<const T*>(a.w_down) + int64_t(e) * H * I;
  const int h0 = blockIdx.x * RROWS + wave_id() * (RROWS / 4);
  float oo = 0.f;
  for (int h = h0; h < h0 + RROWS / 4; ++h) {
    const float o = wave_sum(row_dot<T>(wd + int64_t(h) * I, ve, I));
    oo += o * o;  // the same in every lane
  }
  if (lane_id() == 0) s_red[wave_id()] = oo;
  __syncthreads();
  if (threadIdx.x == 0)
    a.ws_opart[int64_t(e) * gridDim.x + blockIdx.x] =
        double(s_red[0]) + double(s_red[1]) + double(s_red[2]) + double(s_red[3]);
}

// Raw RCR values and the layer-mean normalisation of both tables (one workgroup).
__global__ void tables_finalize_kernel(TablesArgs a) {
  __shared__ double s_mean[2];
  const int nblk = a.H / RROWS;
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
    double s = 0.0;
    for (int c = 0; c < nblk; ++c) s += a.ws_opart[int64_t(e) * nblk + c];
    a.ws_raw_rcr[e] = sqrt(s) / (double(a.ws_qnorm[e]) + double(a.eps));
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    const double* raw = threadIdx.x == 0 ? a.ws_raw_gsp : a.ws_raw_rcr;
    double s = 0.0;
    for (int e = 0; e < a.E; ++e) s += raw[e];
    s_mean[threadIdx.x] = s / a.E;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
    a.a_gsp[e] = float(a.ws_raw_gsp[e] / (s_mean[0] + double(a.eps)));
    a.a_rcr[e] = float(a.ws_raw_rcr[e] / (s_mean[1] + double(a.eps)));
  }
}

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

struct TablesLayout {
  int nb;         // experts per Gram batch
  int ntiles;     // upper-triangular tiles per expert
  size_t off[8];  // wdT, tile partials, mean row, x, ‖q‖, v, row partials, raw values
  size_t total;
};

size_t per_expert_bytes(int H, int I, int dtype) { return size_t(I) * H * (dtype == 1 ? 2 : 4); }

// Workspace carve-up for Gram batches of nb experts.
TablesLayout tables_layout(int E, int H, int I, int dtype, int nb) {
  TablesLayout L;
  L.nb = nb;
  const int nbk = I / GT;
  L.ntiles = nbk * (nbk + 1) / 2;
  const size_t sz[8] = {size_t(nb) * per_expert_bytes(H, I, dtype),
                        size_t(nb) * L.ntiles * 4 * sizeof(double),
                        size_t(H) * sizeof(float),
                        size_t(E) * H * sizeof(float),
                        size_t(E) * sizeof(float),
                        size_t(E) * I * sizeof(float),
                        size_t(E) * (H / RROWS) * sizeof(double),
                        2 * size_t(E) * sizeof(double)};
  size_t o = 0;
  for (int i = 0; i < 8; ++i) {
    L.off[i] = o;
    o += al256(sz[i]);
  }
  L.total = o;
  return L;
}

// Preferred batch: every expert, or as many as WDT_CAP bytes of transposed w_down hold.
int preferred_batch(int E, int H, int I, int dtype) {
  return int(std::max<size_t>(1, std::min<size_t>(size_t(E), WDT_CAP / per_expert_bytes(H, I, dtype))));
}

}  // namespace

size_t tables_workspace_bytes(int E, int H, int I, int dtype, bool minimum) {
  return tables_layout(E, H, I, dtype, minimum ? 1 : preferred_batch(E, H, I, dtype)).total;
}

hipError_t launch_tables(int dtype, TablesArgs a, void* workspace, size_t workspace_bytes, hipStream_t s) {
  int nb = preferred_batch(a.E, a.H, a.I, dtype);
  while (nb > 1 && tables_layout(a.E, a.H, a.I, dtype, nb).total > workspace_bytes) --nb;
  const TablesLayout L = tables_layout(a.E, a.H, a.I, dtype, nb);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  a.ws_wdT = w + L.off[0];
  a.ws_part = reinterpret_cast<double*>(w + L.off[1]);
  a.ws_mean = reinterpret_cast<float*>(w + L.off[2]);
  a.ws_x = reinterpret_cast<float*>(w + L.off[3]);
  a.ws_qnorm = reinterpret_cast<float*>(w + L.off[4]);
  a.ws_v = reinterpret_cast<float*>(w + L.off[5]);
  a.ws_opart = reinterpret_cast<double*>(w + L.off[6]);
  a.ws_raw_gsp = reinterpret_cast<double*>(w + L.off[7]);
  a.ws_raw_rcr = a.ws_raw_gsp + a.E;
  hipError_t err;
#define ACE_LAUNCH(...)                                        \
  do {                                                         \
    hipLaunchKernelGGL(__VA_ARGS__);                           \
    if ((err = hipGetLastError()) != hipSuccess) return err;   \
  } while (0)
  for (int e0 = 0; e0 < a.E; e0 += L.nb) {
    const int nb = std::min(L.nb, a.E - e0);
    const dim3 tgrid(a.I / 64, a.H / 64, nb);
    const int total = nb * L.ntiles;
    const dim3 ggrid(NXCD * ((total + NXCD - 1) / NXCD));
    if (dtype == 1) {
      ACE_LAUNCH(tables_transpose_kernel<bf16_t>, tgrid, dim3(256), 0, s, a, e0);
      ACE_LAUNCH(tables_gram_kernel<bf16_t>, ggrid, dim3(GNTHR), 0, s, a, e0, nb);
    } else {
      ACE_LAUNCH(tables_transpose_kernel<float>, tgrid, dim3(256), 0, s, a, e0);
      ACE_LAUNCH(tables_gram_kernel<float>, ggrid, dim3(GNTHR), 0, s, a, e0, nb);
    }
    ACE_LAUNCH(tables_gsp_reduce_kernel, dim3((nb + 63) / 64), dim3(64), 0, s, a, e0, nb);
  }
  ACE_LAUNCH(tables_rcr_mean_kernel, dim3((a.H + 255) / 256), dim3(256), 0, s, a);
  ACE_LAUNCH(tables_rcr_proto_kernel, dim3(a.E), dim3(256), 0, s, a);
  if (dtype == 1) {
    ACE_LAUNCH(tables_rcr_up_kernel<bf16_t>, dim3(a.I / RROWS, a.E), dim3(256), 0, s, a);
    ACE_LAUNCH(tables_rcr_down_kernel<bf16_t>, dim3(a.H / RROWS, a.E), dim3(256), 0, s, a);
  } else {
    ACE_LAUNCH(tables_rcr_up_kernel<float>, dim3(a.I / RROWS, a.E), dim3(256), 0, s, a);
    ACE_LAUNCH(tables_rcr_down_kernel<float>, dim3(a.H / RROWS, a.E), dim3(256), 0, s, a);
  }
  ACE_LAUNCH(tables_finalize_kernel, dim3(1), dim3(256), 0, s, a);
#undef ACE_LAUNCH
  return hipSuccess;
}

}  // namespace ace
