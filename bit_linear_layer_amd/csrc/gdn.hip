// Gated delta-rule recurrence of a Gated DeltaNet layer, consuming the gate
// epilogue's write strength beta = sigmoid(b) and log-space decay
// g = -exp(A_log) softplus(a + dt_bias) (chatpaper.ai English abstract,
// mechanisms (ii) and (iii); evolve.pub review, "Key claims under review",
// third claim).  Per value head, state S in R^{128 x 128} (rows: value dims,
// columns: key dims):
//     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//     o_t = S_t q_t,
// the published gated delta rule; q/k heads are shared by groups of value
// heads, optionally L2-normalized (q scaled by 128^-1/2).  float32 throughout.
//
// Chunked form (64 tokens per chunk, derived from the update): with
// u_t = beta_t (v_t - exp(g_t) S_{t-1} k_t) the update is
// S_t = exp(g_t) S_{t-1} + u_t k_t^T.  Inside a chunk starting from S0 with
// cumulative decay G_t = exp(g_1 + ... + g_t):
//     (I + M) U = diag(beta) (V - diag(G) K S0^T),
//     M[t][j] = beta_t (G_t / G_j) k_t.k_j  (j < t),
// so U = Ut - Wt S0^T with [Wt | Ut] = (I + M)^-1 diag(beta) [diag(G) K | V];
//     O = diag(G) Q S0^T + A U,  A[t][j] = (G_t / G_j) q_t.k_j  (j <= t),
//     S_end = G_C S0 + U^T diag(G_C / G) K.
// Wt, Ut, A, diag(G) Q and diag(G_C/G) K depend on the chunk only, so one
// kernel computes them for every (key head, chunk) in parallel, sharing k.k^T
// and q.k^T among the value heads of a key head; a second walks
// the chunks in order per (head, 32-row slice of S): the rows of S evolve
// independently, so slices need no communication.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "internal.h"

namespace nvfp4 {

namespace {

using namespace dev;
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;   // head dimension (keys and values)
constexpr int kC = 64;    // tokens per chunk
constexpr int kSlice = 32;  // state rows per scan workgroup
constexpr int kThreads = 256;       // prep workgroup
constexpr int kScanThreads = 512;   // scan workgroup
// LDS row strides, padded so the 16 rows a wave reads at once fall into
// distinct banks (an unpadded 512-byte stride puts them all in one)
constexpr int kP = kD + 4;   // rows of 128 floats
constexpr int kPA = kC + 4;  // rows of 64 floats

// Workspace per (value head, chunk), floats.
constexpr int64_t kWsW = 0;                  // Wt   [64][128]
constexpr int64_t kWsU = kWsW + kC * kD;     // Ut   [64][128]
constexpr int64_t kWsA = kWsU + kC * kD;     // A    [64][64]
constexpr int64_t kWsQ = kWsA + kC * kC;     // diag(G) Q        [64][128]
constexpr int64_t kWsK = kWsQ + kC * kD;     // diag(G_C / G) K  [64][128]
constexpr int64_t kWsG = kWsK + kC * kD;     // G_C (one float, padded to 4)
constexpr int64_t kWsPerChunk = kWsG + 4;

template <int DT>
__device__ inline float load_elem(const void* base, int64_t idx) {
  if constexpr (DT == NVFP4_DTYPE_BF16) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[idx] << 16);
  } else {
    return reinterpret_cast<const float*>(base)[idx];
  }
}

// 32 consecutive elements (a quarter of a 128-wide head row) as floats, with
// 16-byte loads (rows are 16-byte aligned); zeros when !valid.
template <int DT>
__device__ inline void load32(const void* base, int64_t elem, bool valid, float v[32]) {
  if constexpr (DT == NVFP4_DTYPE_BF16) {
    uint4 w[4];
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
    if (valid) {  // rows past the end are never read
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = src[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * j + 2 * e] = __uint_as_float(x[e] << 16);
        v[8 * j + 2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    float4 f[8];
    if (valid) {  // rows past the end are never read
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = src[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[4 * j] = f[j].x; v[4 * j + 1] = f[j].y; v[4 * j + 2] = f[j].z; v[4 * j + 3] = f[j].w;
    }
  }
}

__device__ inline void store32(float* dst, const float v[32]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    reinterpret_cast<float4*>(dst)[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
}

// Inclusive prefix sum over the 64 lanes of one wave.
__device__ inline float wave_prefix_sum(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// One workgroup per (chunk, key head): the q/k rows, k.k^T and q.k^T once,
// then, for each value head reading that key head, its decay and write
// strength applied and the forward substitution.
template <int DT>
__global__ __launch_bounds__(kThreads) void gdn_prep_kernel(GdnArgs p, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) float sk[kC][kP];  // k rows (normalized)
  __shared__ __attribute__((aligned(16))) float sq[kC][kP];  // q rows (normalized, scaled)
  __shared__ __attribute__((aligned(16))) float sw[kC][kP];  // right-hand sides / solution, Wt half
  __shared__ __attribute__((aligned(16))) float sv[kC][kP];  // right-hand sides / solution, Ut half
  __shared__ __attribute__((aligned(16))) float sm[kC][kPA];  // M (strictly lower)
  __shared__ float sgam[kC];     // cumulative log decay
  __shared__ float sbeta[kC];

  const int chunk = blockIdx.x, hk = blockIdx.y;
  const int rep = p.hv / p.hk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)chunk * kC;

  // q, k rows of the chunk (zero beyond T: such tokens have beta = 0, g = 0
  // and leave the state unchanged); thread -> row tid/4, quarter tid%4, all
  // loads issued before use; L2 norms reduced over the row's 4 threads
  {
    const int t = tid >> 2, part = tid & 3;
    const int64_t tt = t0 + t;
    const bool valid = tt < p.T;
    float kr[32], qr[32];
    load32<DT>(p.k, tt * p.ld_k + (int64_t)hk * kD + part * 32, valid, kr);
    load32<DT>(p.q, tt * p.ld_q + (int64_t)hk * kD + part * 32, valid, qr);
    if (p.normalize) {
      float sk2 = 0.0f, sq2 = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        sk2 += kr[e] * kr[e];
        sq2 += qr[e] * qr[e];
      }
      sk2 += __shfl_xor(sk2, 1);
      sk2 += __shfl_xor(sk2, 2);
      sq2 += __shfl_xor(sq2, 1);
      sq2 += __shfl_xor(sq2, 2);
      const float ik = 1.0f / fmaxf(sqrtf(sk2), 1e-30f);
      const float iq = 0.08838834764831845f / fmaxf(sqrtf(sq2), 1e-30f);  // 128^-1/2 / |q|
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        kr[e] *= ik;
        qr[e] *= iq;
      }
    }
    store32(&sk[t][part * 32], kr);
    store32(&sq[t][part * 32], qr);
  }
  __syncthreads();

  // k_t.k_j and q_t.k_j: thread -> row t, 16 columns, kept in registers for
  // every value head of the group
  const int mt = tid >> 2, j0 = (tid & 3) * 16;
  float km[16], qm[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) km[i] = qm[i] = 0.0f;
  for (int d = 0; d < kD; d += 4) {
    const float4 kt = *reinterpret_cast<const float4*>(&sk[mt][d]);
    const float4 qt = *reinterpret_cast<const float4*>(&sq[mt][d]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 kj = *reinterpret_cast<const float4*>(&sk[j0 + i][d]);
      km[i] += kt.x * kj.x + kt.y * kj.y + kt.z * kj.z + kt.w * kj.w;
      qm[i] += qt.x * kj.x + qt.y * kj.y + qt.z * kj.z + qt.w * kj.w;
    }
  }

  for (int hr = 0; hr < rep; ++hr) {
    const int h = hk * rep + hr;
    float* out = ws + ((int64_t)h * p.n_chunks + chunk) * kWsPerChunk;
    if (wave == 0) {
      const int64_t tt = t0 + lane;
      float b = 0.0f, g = 0.0f;
      if (tt < p.T) {
        b = load_elem<DT>(p.beta, tt * p.ld_beta + h);
        g = load_elem<DT>(p.g, tt * p.ld_g + h);
      }
      sbeta[lane] = b;
      sgam[lane] = wave_prefix_sum(g, lane);
    }
    // this head's v rows, issued early
    float vr[32];
    {
      const int t = tid >> 2, part = tid & 3;
      load32<DT>(p.v, (t0 + t) * p.ld_v + (int64_t)h * kD + part * 32, t0 + t < p.T, vr);
    }
    __syncthreads();  // beta, gamma of this head; every read of the previous head's buffers done

    // M[t][j] = beta_t exp(gam_t - gam_j) k_t.k_j (j < t) and
    // A[t][j] = exp(gam_t - gam_j) q_t.k_j (j <= t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + i;
      const float dec = expf(sgam[mt] - sgam[j]);
      sm[mt][j] = j < mt ? sbeta[mt] * dec * km[i] : 0.0f;
      out[kWsA + mt * kC + j] = j <= mt ? dec * qm[i] : 0.0f;
    }
    // diag(G) Q, diag(G_C / G) K, G_C, and the right-hand sides
    // beta diag(G) K and beta V
    const float gc = sgam[kC - 1];
    {
      const int t = tid >> 2, part = tid & 3;
      const float eg = expf(sgam[t]), egc = expf(gc - sgam[t]), bt = sbeta[t];
#pragma unroll
      for (int e = 0; e < 32; e += 4) {
        const int d = part * 32 + e;
        const float4 kv = *reinterpret_cast<const float4*>(&sk[t][d]);
        const float4 qv = *reinterpret_cast<const float4*>(&sq[t][d]);
        *reinterpret_cast<float4*>(out + kWsQ + t * kD + d) = make_float4(eg * qv.x, eg * qv.y, eg * qv.z, eg * qv.w);
        *reinterpret_cast<float4*>(out + kWsK + t * kD + d) =
            make_float4(egc * kv.x, egc * kv.y, egc * kv.z, egc * kv.w);
        const float s = bt * eg;
        *reinterpret_cast<float4*>(&sw[t][d]) = make_float4(s * kv.x, s * kv.y, s * kv.z, s * kv.w);
        *reinterpret_cast<float4*>(&sv[t][d]) =
            make_float4(bt * vr[e], bt * vr[e + 1], bt * vr[e + 2], bt * vr[e + 3]);
      }
    }
    if (tid == 0) out[kWsG] = expf(gc);
    __syncthreads();

    // [Wt | Ut] = (I + M)^-1 [rhs] by forward substitution in place: thread c
    // owns column c of [sw | sv] (a wave's columns are all of one kind); 16
    // rows at a time in registers, earlier rows read back final from LDS, M
    // read as a broadcast
    {
      const bool wcol = tid < kD;
      const int cc = tid & (kD - 1);
      float* col = wcol ? &sw[0][cc] : &sv[0][cc];  // element t at col[t * kP]
      for (int b0 = 0; b0 < kC; b0 += 16) {
        float r[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) r[i] = col[(b0 + i) * kP];
        for (int j = 0; j < b0; j += 4) {  // b0 is a multiple of 16
          const float y0 = col[j * kP], y1 = col[(j + 1) * kP], y2 = col[(j + 2) * kP], y3 = col[(j + 3) * kP];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float4 m = *reinterpret_cast<const float4*>(&sm[b0 + i][j]);
            r[i] -= m.x * y0 + m.y * y1 + m.z * y2 + m.w * y3;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
          for (int jj = 0; jj < i; ++jj) r[i] -= sm[b0 + i][b0 + jj] * r[jj];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) col[(b0 + i) * kP] = r[i];
      }
      float* dst = out + (wcol ? kWsW : kWsU);
      for (int t = 0; t < kC; ++t) dst[t * kD + cc] = col[t * kP];
    }
  }
}

// One workgroup per (value head, 32-row slice of S); chunks in order.  The
// three products of a chunk run on v_mfma_f32_16x16x4f32 (fp32 in, fp32
// accumulate; lane l supplies A[l%16][l/16] and B[l/16][l%16] and holds
// D[4(l/16)+r][l%16]):
//   wave w: P = Wt S^T and O = diag(G) Q S^T for the 16x16 tile
//           (t: 16(w/2).., c: 16(w%2)..), U = Ut - P, then O += A U;
//   wave w: S[c][16w..16w+15] = G_C S + U^T diag(G_C/G) K for both 16-row
//           halves of the slice.
// The next chunk's data is loaded into registers while one is computed.
constexpr int kPK = kD + 16;        // k rows, read down a column by 4 lane groups
constexpr int kPU = kSlice + 16;    // U tile [64][32]

// A chunk's data in registers: thread tid holds 4-float group number
// tid + 512 i of Wt, diag(G) Q, diag(G_C/G) K ([64][128]) and of A
// ([64][64]), and the 4 elements of Ut its wave's U tile needs.  Native
// vector types: arrays of HIP's float4 class stay in scratch memory.
__device__ __attribute__((always_inline)) inline void scan_load(const float* in, int tid, int uoff, floatx4 (&w)[4],
                                                                  floatx4 (&q)[4], floatx4 (&k)[4], floatx4 (&a)[2],
                                                                  float (&u)[4], float& gc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[i] = reinterpret_cast<const floatx4*>(in + kWsW)[tid + i * kScanThreads];
    q[i] = reinterpret_cast<const floatx4*>(in + kWsQ)[tid + i * kScanThreads];
    k[i] = reinterpret_cast<const floatx4*>(in + kWsK)[tid + i * kScanThreads];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) a[i] = reinterpret_cast<const floatx4*>(in + kWsA)[tid + i * kScanThreads];
#pragma unroll
  for (int r = 0; r < 4; ++r) u[r] = in[kWsU + uoff + r * kD];
  gc = in[kWsG];
}

template <int ODT>
__global__ __launch_bounds__(kScanThreads) void gdn_scan_kernel(GdnArgs p, const float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) float sS[kSlice][kP];  // this slice of the state
  __shared__ __attribute__((aligned(16))) float sW[kC][kP];      // Wt
  __shared__ __attribute__((aligned(16))) float sQ[kC][kP];      // diag(G) Q
  __shared__ __attribute__((aligned(16))) float sK[kC][kPK];     // diag(G_C/G) K
  __shared__ __attribute__((aligned(16))) float sA[kC][kPA];
  __shared__ float sU[kC][kPU];

  // workgroups of one head on one XCD (ids are dealt to the 8 XCDs
  // round-robin), so its slices share the L2 copy of the chunk data
  constexpr int nsl = kD / kSlice;
  const int bid = blockIdx.x;
  const int x = bid % 8, r8 = bid / 8;
  const int h = (r8 / nsl) * 8 + x, sl = r8 % nsl;
  if (h >= p.hv) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int ti = wave >> 1, tj = wave & 1;  // U / O tile
  const int row0 = sl * kSlice;
  const float* base = ws + (int64_t)h * p.n_chunks * kWsPerChunk;

  const int uoff = (16 * ti + 4 * lk) * kD + row0 + 16 * tj + li;  // this lane's Ut elements
  floatx4 nw[4], nq[4], nk[4], na[2];
  float nu[4], ngc;
  float cu[4], cgc;

  for (int i = tid; i < kSlice * kD; i += kScanThreads) {
    const int c = i / kD, d = i % kD;
    sS[c][d] = p.s0 != nullptr ? p.s0[((int64_t)h * kD + row0 + c) * kD + d] : 0.0f;
  }
  scan_load(base, tid, uoff, nw, nq, nk, na, nu, ngc);

  for (int chunk = 0; chunk < p.n_chunks; ++chunk) {
    // this chunk's data: registers -> LDS (every read of the previous
    // chunk's data is behind the barrier at the end of the iteration)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + i * kScanThreads;
      const int rr = f / (kD / 4), cc = (f % (kD / 4)) * 4;
      *reinterpret_cast<floatx4*>(&sW[rr][cc]) = nw[i];
      *reinterpret_cast<floatx4*>(&sQ[rr][cc]) = nq[i];
      *reinterpret_cast<floatx4*>(&sK[rr][cc]) = nk[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = tid + i * kScanThreads;
      *reinterpret_cast<floatx4*>(&sA[f / (kC / 4)][(f % (kC / 4)) * 4]) = na[i];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) cu[r] = nu[r];
    cgc = ngc;
    __syncthreads();
    // the next chunk's loads fly while this one is computed; unconditional
    // (the last chunk reloads itself): a load under a branch makes the
    // compiler wait for it where the paths join
    scan_load(base + (int64_t)(chunk + 1 < p.n_chunks ? chunk + 1 : chunk) * kWsPerChunk, tid, uoff, nw, nq, nk, na,
              nu, ngc);

    // P = Wt S^T and O = diag(G) Q S^T on this wave's tile
    floatx4 accp = {0.0f, 0.0f, 0.0f, 0.0f}, acco = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int k = 0; k < kD / 4; ++k) {
      const float bs = sS[16 * tj + li][4 * k + lk];
      accp = __builtin_amdgcn_mfma_f32_16x16x4f32(sW[16 * ti + li][4 * k + lk], bs, accp, 0, 0, 0);
      acco = __builtin_amdgcn_mfma_f32_16x16x4f32(sQ[16 * ti + li][4 * k + lk], bs, acco, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) sU[16 * ti + 4 * lk + q][16 * tj + li] = cu[q] - accp[q];
    __syncthreads();
    // O += A U over the key positions j <= t (A is lower triangular)
    for (int k = 0; k < 4 * (ti + 1); ++k)
      acco = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * ti + li][4 * k + lk], sU[4 * k + lk][16 * tj + li], acco,
                                                  0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t tt = (int64_t)chunk * kC + 16 * ti + 4 * lk + q;
      if (tt < p.T) {
        const int64_t idx = tt * p.ld_o + (int64_t)h * kD + row0 + 16 * tj + li;
        if constexpr (ODT == NVFP4_DTYPE_BF16)
          reinterpret_cast<uint16_t*>(p.o)[idx] = (uint16_t)f32_to_bf16_bits(acco[q]);
        else
          reinterpret_cast<float*>(p.o)[idx] = acco[q];
      }
    }
    // S[c][16w + j] = G_C S + U^T diag(G_C/G) K: each wave reads and writes
    // only its own 16 columns of the slice, after every wave's reads of S
    // above (the barrier after U)
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      floatx4 acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = cgc * sS[16 * tc + 4 * lk + q][16 * wave + li];
#pragma unroll 8
      for (int k = 0; k < kC / 4; ++k)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sU[4 * k + lk][16 * tc + li], sK[4 * k + lk][16 * wave + li], acc,
                                                   0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) sS[16 * tc + 4 * lk + q][16 * wave + li] = acc[q];
    }
    __syncthreads();  // every read of this chunk's data and of the new S is done
  }
  if (p.s_final != nullptr)
    for (int i = tid; i < kSlice * kD; i += kScanThreads) {
      const int c = i / kD, d = i % kD;
      p.s_final[((int64_t)h * kD + row0 + c) * kD + d] = sS[c][d];
    }
}

}  // namespace

size_t gdn_workspace_floats(int64_t T, int hv) {
  const int64_t chunks = (T + kC - 1) / kC;
  return (size_t)(chunks * hv * kWsPerChunk);
}

hipError_t launch_gdn(const GdnArgs& p, float* ws, hipStream_t s) {
  const dim3 prep((unsigned)p.n_chunks, (unsigned)p.hk);
  if (p.in_dtype == NVFP4_DTYPE_BF16)
    gdn_prep_kernel<NVFP4_DTYPE_BF16><<<prep, kThreads, 0, s>>>(p, ws);
  else
    gdn_prep_kernel<NVFP4_DTYPE_F32><<<prep, kThreads, 0, s>>>(p, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nsl = kD / kSlice;
  const unsigned blocks = (unsigned)(((p.hv + 7) / 8) * 8 * nsl);
  if (p.o_dtype == NVFP4_DTYPE_BF16)
    gdn_scan_kernel<NVFP4_DTYPE_BF16><<<blocks, kScanThreads, 0, s>>>(p, ws);
  else
    gdn_scan_kernel<NVFP4_DTYPE_F32><<<blocks, kScanThreads, 0, s>>>(p, ws);
  return hipGetLastError();
}

}  // namespace nvfp4
