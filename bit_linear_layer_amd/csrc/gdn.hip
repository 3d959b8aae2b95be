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
// independently, so slices need no communication.  The normalized q and k
// are stored once per key head and chunk, with the per-token factors G_t
// and G_C / G_t per value head: the scan forms diag(G) Q and
// (diag(G_C/G) K)^T itself with the same float32 products, so the workspace
// written and read back is 29 % smaller (44 % per value head).
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
constexpr int kScanThreads = 512;   // scan workgroup
// LDS row strides, padded so the 16 rows a wave reads at once fall into
// distinct banks (an unpadded 512-byte stride puts them all in one)
constexpr int kP = kD + 4;   // rows of 128 floats
constexpr int kPA = kC + 4;  // rows of 64 floats

// Workspace, floats: per (value head, chunk) a block of kWsPerChunk, all
// value heads first; after them per (key head, chunk) a block of
// kWsPerKeyChunk (room is reserved for as many key heads as value heads, so
// the size depends on tokens and value heads only).
constexpr int64_t kWsW = 0;                  // Wt   [64][128]
constexpr int64_t kWsU = kWsW + kC * kD;     // Ut   [64][128]
constexpr int64_t kWsA = kWsU + kC * kD;     // A    [64][64]
constexpr int64_t kWsEG = kWsA + kC * kC;    // G_t = exp(cumulative log decay)  [64]
constexpr int64_t kWsEC = kWsEG + kC;        // G_C / G_t  [64]
constexpr int64_t kWsG = kWsEC + kC;         // G_C (one float, padded to 4)
constexpr int64_t kWsPerChunk = kWsG + 4;
constexpr int64_t kWsQN = 0;                 // normalized (and 128^-1/2-scaled) q  [64][128]
constexpr int64_t kWsKT = kWsQN + kC * kD;   // normalized k, transposed  [128][64]
constexpr int64_t kWsPerKeyChunk = kWsKT + kC * kD;

__host__ __device__ inline int64_t key_block(int64_t hv, int64_t n_chunks, int64_t hk, int64_t chunk) {
  return hv * n_chunks * kWsPerChunk + (hk * n_chunks + chunk) * kWsPerKeyChunk;
}

template <int DT>
__device__ inline float load_elem(const void* base, int64_t idx) {
  if constexpr (DT == NVFP4_DTYPE_BF16) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[idx] << 16);
  } else {
    return reinterpret_cast<const float*>(base)[idx];
  }
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

// 16 consecutive elements of a head row as floats, unconditionally (the
// caller clamps the row into range): two 16-byte loads (bf16) or four (f32).
template <int DT>
__device__ inline void load16(const void* base, int64_t elem, float v[16]) {
  if constexpr (DT == NVFP4_DTYPE_BF16) {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
    const uint4 w0 = src[0], w1 = src[1];
    const uint32_t x[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[2 * e] = __uint_as_float(x[e] << 16);
      v[2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
    }
  } else {
    const floatx4* src = reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(base) + elem);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const floatx4 f = src[j];
      v[4 * j] = f[0]; v[4 * j + 1] = f[1]; v[4 * j + 2] = f[2]; v[4 * j + 3] = f[3];
    }
  }
}

constexpr int kPrepThreads = 512;  // 8 waves

// One workgroup per (chunk, key head).  Everything but the 16x16 diagonal
// blocks of the triangular inverse runs on v_mfma_f32_16x16x4f32.  Inside a
// product's 16-wide K block the lane group g = lane/16 takes k = 4g + s at
// MFMA step s (any order of k gives the same sum), so an A operand is one
// 16-byte LDS read per 4 steps and a product's accumulator (lane holds
// D[4g + r][lane%16]) is directly the B operand of the next product.
//   1. q, k rows, L2-normalized, into LDS; K K^T and Q K^T (waves 0-3 and
//      4-7, one 16-row block each) stay in registers for every value head.
//   2. per value head: M = (beta_t G_t/G_j k_t.k_j)_{j<t} into LDS, A out;
//      T = (I + M)^-1 block by block -- diagonal 16x16 blocks by forward
//      substitution, then T_ij = -T_ii sum_{i>k>=j} M_ik T_kj one block
//      diagonal at a time; Wt = T diag(beta G) K and Ut = T diag(beta) V as
//      block-triangular products.
// The next head's v, beta, g are loaded before this head's stores, so
// waiting for them never waits for the stores (one counter covers both).
template <int DT>
__global__ __launch_bounds__(kPrepThreads) void gdn_prep_kernel(GdnArgs p, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) float sk[kC][kP];   // k rows (normalized)
  __shared__ __attribute__((aligned(16))) float sq[kC][kP];   // q rows (normalized, scaled)
  __shared__ __attribute__((aligned(16))) float sv[kC][kP];   // v rows of the current head
  __shared__ __attribute__((aligned(16))) float sm[kC][kPA];  // M (strictly lower)
  __shared__ __attribute__((aligned(16))) float st[kC][kPA];  // T = (I + M)^-1 (lower blocks)
  __shared__ __attribute__((aligned(16))) float sgam[kC];     // cumulative log decay
  __shared__ __attribute__((aligned(16))) float sbeta[kC];    // beta_j
  __shared__ __attribute__((aligned(16))) float scw[kC];      // beta_j G_j
  __shared__ __attribute__((aligned(16))) float segc[kC];     // G_C / G_t

  const int chunk = blockIdx.x, hk = blockIdx.y;
  const int rep = p.hv / p.hk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)chunk * kC;
  const int rt = tid >> 3, part = tid & 7;  // row-wise work: row rt, elements 16 part ..
  const bool rvalid = t0 + rt < p.T;
  const int64_t rrow = rvalid ? t0 + rt : p.T - 1;       // clamped, always a valid address
  const int64_t lrow = t0 + lane < p.T ? t0 + lane : p.T - 1;

  // the first head's v, beta, g go out with q and k
  float vn[16], bn = 0.0f, gn = 0.0f;
  auto load_head = [&](int h) {
    load16<DT>(p.v, rrow * p.ld_v + (int64_t)h * kD + part * 16, vn);
    bn = load_elem<DT>(p.beta, lrow * p.ld_beta + h);
    gn = load_elem<DT>(p.g, lrow * p.ld_g + h);
  };
  load_head(hk * rep);
  {
    float kr[16], qr[16];
    load16<DT>(p.k, rrow * p.ld_k + (int64_t)hk * kD + part * 16, kr);
    load16<DT>(p.q, rrow * p.ld_q + (int64_t)hk * kD + part * 16, qr);
    float ik = rvalid ? 1.0f : 0.0f, iq = ik;  // rows past T are zero
    if (p.normalize) {
      float sk2 = 0.0f, sq2 = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sk2 += kr[e] * kr[e];
        sq2 += qr[e] * qr[e];
      }
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) {
        sk2 += __shfl_xor(sk2, off);
        sq2 += __shfl_xor(sq2, off);
      }
      ik *= 1.0f / fmaxf(sqrtf(sk2), 1e-30f);
      iq *= 0.08838834764831845f / fmaxf(sqrtf(sq2), 1e-30f);  // 128^-1/2 / |q|
    }
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      *reinterpret_cast<floatx4*>(&sk[rt][part * 16 + e]) =
          floatx4{kr[e] * ik, kr[e + 1] * ik, kr[e + 2] * ik, kr[e + 3] * ik};
      *reinterpret_cast<floatx4*>(&sq[rt][part * 16 + e]) =
          floatx4{qr[e] * iq, qr[e + 1] * iq, qr[e + 2] * iq, qr[e + 3] * iq};
    }
  }
  __syncthreads();
  {
    // the normalized q rows and k^T (key dimension major: the scan reads it
    // down the token axis) of this key head and chunk
    float* kout = ws + key_block(p.hv, p.n_chunks, hk, chunk);
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *reinterpret_cast<floatx4*>(kout + kWsQN + rt * kD + part * 16 + e) =
          *reinterpret_cast<const floatx4*>(&sq[rt][part * 16 + e]);
    const int d = tid >> 2, tq = (tid & 3) * 16;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const int t = tq + e;
      *reinterpret_cast<floatx4*>(kout + kWsKT + d * kC + t) = floatx4{sk[t][d], sk[t + 1][d], sk[t + 2][d], sk[t + 3][d]};
    }
  }

  // K K^T (waves 0-3) or Q K^T (waves 4-7), rows 16 rb.., all 64 columns:
  // gram[cb][r] = (X K^T)[16 rb + 4 lg + r][16 cb + li]
  const int gmat = wave >> 2, rb = wave & 3;
  floatx4 gram[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) gram[cb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  {
    const float* xrow = gmat ? &sq[16 * rb + li][0] : &sk[16 * rb + li][0];
#pragma unroll 2
    for (int k0 = 0; k0 < kD; k0 += 16) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(xrow + k0 + 4 * lg);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const floatx4 b = *reinterpret_cast<const floatx4*>(&sk[16 * cb + li][k0 + 4 * lg]);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) gram[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s2], b[s2], gram[cb], 0, 0, 0);
      }
    }
  }

  for (int hr = 0; hr < rep; ++hr) {
    const int h = hk * rep + hr;
    float* out = ws + ((int64_t)h * p.n_chunks + chunk) * kWsPerChunk;
    __syncthreads();  // every read of the previous head's sv, sm, st, sgam, sbeta, scw is done
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *reinterpret_cast<floatx4*>(&sv[rt][part * 16 + e]) =
          rvalid ? floatx4{vn[e], vn[e + 1], vn[e + 2], vn[e + 3]} : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (wave == 0) {
      const bool ok = t0 + lane < p.T;  // tokens past T: beta = 0, g = 0
      const float b = ok ? bn : 0.0f;
      const float gam = wave_prefix_sum(ok ? gn : 0.0f, lane);
      const float eg = expf(gam), ec = expf(__shfl(gam, 63) - gam);
      sbeta[lane] = b;
      sgam[lane] = gam;
      scw[lane] = b * eg;
      segc[lane] = ec;
      out[kWsEG + lane] = eg;
      out[kWsEC + lane] = ec;
    }
    __syncthreads();
    // the next head's operands (the last head reloads itself) ahead of this
    // head's stores
    load_head(hr + 1 < rep ? h + 1 : h);

    // M into LDS (waves 0-3), A out (waves 4-7)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * rb + 4 * lg + r;
      const float gt = sgam[t], bt = sbeta[t];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int j = 16 * cb + li;
        const float dec = expf(gt - sgam[j]);
        if (gmat == 0)
          sm[t][j] = j < t ? bt * dec * gram[cb][r] : 0.0f;
        else
          out[kWsA + t * kC + j] = j <= t ? dec * gram[cb][r] : 0.0f;
      }
    }
    if (tid == 0) out[kWsG] = expf(sgam[kC - 1]);  // G_C
    __syncthreads();  // M complete

    // diagonal blocks of T: lane (block i, column c) solves (I + M_ii) x = e_c
    if (wave == 0) {
      const int i = lane >> 4, c = lane & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = r == c ? 1.0f : 0.0f;
#pragma unroll
        for (int jj = 0; jj < r; ++jj) v -= sm[16 * i + r][16 * i + jj] * x[jj];
        x[r] = v;
        st[16 * i + r][16 * i + c] = v;
      }
    }
    __syncthreads();
    // off-diagonal blocks, one block diagonal d at a time: T_ij = -T_ii X,
    // X = sum_{k=j}^{i-1} M_ik T_kj
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      if (wave < 4 - d) {
        const int i = wave + d, j = wave;
        floatx4 x = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int kb = j; kb < i; ++kb) {
          const floatx4 a = *reinterpret_cast<const floatx4*>(&sm[16 * i + li][16 * kb + 4 * lg]);
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s2], st[16 * kb + 4 * lg + s2][16 * j + li], x, 0, 0, 0);
        }
        floatx4 y = {0.0f, 0.0f, 0.0f, 0.0f};
        const floatx4 a = *reinterpret_cast<const floatx4*>(&st[16 * i + li][16 * i + 4 * lg]);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) y = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s2], x[s2], y, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) st[16 * i + 4 * lg + r][16 * j + li] = -y[r];
      }
      __syncthreads();
    }

    // Wt = T diag(beta G) K (waves 0-3), Ut = T diag(beta) V (waves 4-7);
    // wave w owns column blocks 2(w%4), 2(w%4)+1, all four row blocks
    {
      const int pm = wave >> 2, cb0 = 32 * (wave & 3);
      const float(*src)[kP] = pm ? sv : sk;
      const float* coef = pm ? sbeta : scw;
      float* dst = out + (pm ? kWsU : kWsW);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        floatx4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int jb = 0; jb <= i; ++jb) {
          const floatx4 a = *reinterpret_cast<const floatx4*>(&st[16 * i + li][16 * jb + 4 * lg]);
          const floatx4 cf = *reinterpret_cast<const floatx4*>(&coef[16 * jb + 4 * lg]);
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const int j = 16 * jb + 4 * lg + s2;
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s2], cf[s2] * src[j][cb0 + li], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s2], cf[s2] * src[j][cb0 + 16 + li], acc1, 0, 0, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * i + 4 * lg + r;
          dst[t * kD + cb0 + li] = acc0[r];
          dst[t * kD + cb0 + 16 + li] = acc1[r];
        }
      }
    }
  }
}

// One workgroup per (value head, 32-row slice of S); chunks in order.  The
// three products of a chunk run on v_mfma_f32_16x16x4f32 (fp32 in, fp32
// accumulate; lane l supplies A[l%16][l/16] and B[l/16][l%16] and holds
// D[4(l/16)+r][l%16]); inside each 16-wide K block lane group l/16 takes
// k = 4(l/16) + s at step s, so operands are 16-byte LDS reads (U is kept
// transposed, K^ arrives transposed):
//   wave w: P = Wt S^T and O = diag(G) Q S^T for the 16x16 tile
//           (t: 16(w/2).., c: 16(w%2)..), U = Ut - P, then O += A U;
//   wave w: S[c][16w..16w+15] = G_C S + U^T diag(G_C/G) K for both 16-row
//           halves of the slice.
// The next chunk's data is loaded into registers while one is computed.

// A chunk's data in registers: thread tid holds 4-float group number
// tid + 512 i of Wt, diag(G) Q, diag(G_C/G) K ([64][128]) and of A
// ([64][64]), and the 4 elements of Ut its wave's U tile needs.  Native
// vector types: arrays of HIP's float4 class stay in scratch memory.
// A chunk's data in registers, in two halves loaded at different points:
// Wt and diag(G) Q (read by the first phase of a step), and K^T, A, the
// lane's Ut elements and G_C (read by the second).  Thread tid holds 4-float
// groups tid + 512 i of each array.  Native vector types: arrays of HIP's
// float4 class stay in scratch memory.
__device__ __attribute__((always_inline)) inline void scan_load_wq(const float* in, const float* kin, int tid,
                                                                     floatx4 (&w)[4], floatx4 (&q)[4],
                                                                     float (&eg)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = tid + i * kScanThreads;
    w[i] = reinterpret_cast<const floatx4*>(in + kWsW)[f];
    q[i] = reinterpret_cast<const floatx4*>(kin + kWsQN)[f];
    eg[i] = in[kWsEG + f / (kD / 4)];  // the row (token) of q's group
  }
}
__device__ __attribute__((always_inline)) inline void scan_load_ka(const float* in, const float* kin, int tid, int uoff,
                                                                     floatx4 (&k)[4], floatx4 (&ec)[4],
                                                                     floatx4 (&a)[2], float (&u)[4], float& gc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = tid + i * kScanThreads;
    k[i] = reinterpret_cast<const floatx4*>(kin + kWsKT)[f];
    ec[i] = *reinterpret_cast<const floatx4*>(in + kWsEC + (f % (kC / 4)) * 4);  // the group's 4 tokens
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
  __shared__ __attribute__((aligned(16))) float sKT[kD][kPA];    // (diag(G_C/G) K)^T
  __shared__ __attribute__((aligned(16))) float sA[kC][kPA];
  __shared__ __attribute__((aligned(16))) float sUT[kSlice][kPA];  // U^T: slice rows x tokens

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
  const float* kbase = ws + key_block(p.hv, p.n_chunks, h / (p.hv / p.hk), 0);
  const int last = p.n_chunks - 1;

  const int uoff = (16 * ti + 4 * lk) * kD + row0 + 16 * tj + li;  // this lane's Ut elements
  floatx4 nw[4], nq[4], nk[4], nec[4], na[2];
  float neg[4], nu[4], ngc;

  auto put_wq = [&]() {  // Wt, diag(G) Q registers -> LDS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + i * kScanThreads;
      const int rr = f / (kD / 4), cc = (f % (kD / 4)) * 4;
      *reinterpret_cast<floatx4*>(&sW[rr][cc]) = nw[i];
      *reinterpret_cast<floatx4*>(&sQ[rr][cc]) = nq[i] * neg[i];
    }
  };
  auto put_ka = [&]() {  // (diag(G_C/G) K)^T, A registers -> LDS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = tid + i * kScanThreads;
      *reinterpret_cast<floatx4*>(&sKT[f / (kC / 4)][(f % (kC / 4)) * 4]) = nk[i] * nec[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = tid + i * kScanThreads;
      *reinterpret_cast<floatx4*>(&sA[f / (kC / 4)][(f % (kC / 4)) * 4]) = na[i];
    }
  };

  for (int i = tid; i < kSlice * kD; i += kScanThreads) {
    const int c = i / kD, d = i % kD;
    sS[c][d] = p.s0 != nullptr ? p.s0[((int64_t)h * kD + row0 + c) * kD + d] : 0.0f;
  }
  scan_load_wq(base, kbase, tid, nw, nq, neg);
  scan_load_ka(base, kbase, tid, uoff, nk, nec, na, nu, ngc);
  put_wq();
  __syncthreads();

  // Two barriers per chunk.  Phase 1 reads Wt, diag(G) Q and S; phase 2
  // reads A, K^T, U and writes S.  So K^T and A of this chunk go to LDS at
  // the end of phase 1 and Wt, diag(G) Q of the next chunk at the end of
  // phase 2, each half loaded into registers one phase earlier.  Loads are
  // unconditional (the last chunk reloads itself): a load under a branch
  // makes the compiler wait for it where the paths join.
  for (int chunk = 0; chunk < p.n_chunks; ++chunk) {
    const float* nxt = base + (int64_t)min(chunk + 1, last) * kWsPerChunk;
    const float* knxt = kbase + (int64_t)min(chunk + 1, last) * kWsPerKeyChunk;
    // ---- phase 1
    scan_load_wq(nxt, knxt, tid, nw, nq, neg);
    // P = Wt S^T and O = diag(G) Q S^T on this wave's tile; inside each
    // 16-wide K block the lane group lk takes k = 4 lk + s at step s (any
    // order of k gives the same sum), so each operand is one 16-byte read
    floatx4 accp = {0.0f, 0.0f, 0.0f, 0.0f}, acco = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < kD / 16; ++kb) {
      const floatx4 bs = *reinterpret_cast<const floatx4*>(&sS[16 * tj + li][16 * kb + 4 * lk]);
      const floatx4 aw = *reinterpret_cast<const floatx4*>(&sW[16 * ti + li][16 * kb + 4 * lk]);
      const floatx4 aq = *reinterpret_cast<const floatx4*>(&sQ[16 * ti + li][16 * kb + 4 * lk]);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        accp = __builtin_amdgcn_mfma_f32_16x16x4f32(aw[s2], bs[s2], accp, 0, 0, 0);
        acco = __builtin_amdgcn_mfma_f32_16x16x4f32(aq[s2], bs[s2], acco, 0, 0, 0);
      }
    }
    *reinterpret_cast<floatx4*>(&sUT[16 * tj + li][16 * ti + 4 * lk]) =
        floatx4{nu[0] - accp[0], nu[1] - accp[1], nu[2] - accp[2], nu[3] - accp[3]};
    put_ka();
    __syncthreads();  // U, K^T, A of this chunk in LDS; every read of Wt, Q, S done
    // ---- phase 2
    const float gc = ngc;
    scan_load_ka(nxt, knxt, tid, uoff, nk, nec, na, nu, ngc);
    // O += A U over key blocks kb <= ti (A is lower triangular)
    for (int kb = 0; kb <= ti; ++kb) {
      const floatx4 aa = *reinterpret_cast<const floatx4*>(&sA[16 * ti + li][16 * kb + 4 * lk]);
      const floatx4 bu = *reinterpret_cast<const floatx4*>(&sUT[16 * tj + li][16 * kb + 4 * lk]);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) acco = __builtin_amdgcn_mfma_f32_16x16x4f32(aa[s2], bu[s2], acco, 0, 0, 0);
    }
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
    // only its own 16 columns of the slice
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      floatx4 acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = gc * sS[16 * tc + 4 * lk + q][16 * wave + li];
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        const floatx4 au = *reinterpret_cast<const floatx4*>(&sUT[16 * tc + li][16 * kb + 4 * lk]);
        const floatx4 bk = *reinterpret_cast<const floatx4*>(&sKT[16 * wave + li][16 * kb + 4 * lk]);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(au[s2], bk[s2], acc, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sS[16 * tc + 4 * lk + q][16 * wave + li] = acc[q];
    }
    put_wq();         // the next chunk's Wt, diag(G) Q
    __syncthreads();  // new S, next Wt and Q in LDS; every read of this chunk's A, K^T, U done
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
  return (size_t)(chunks * hv * (kWsPerChunk + kWsPerKeyChunk));
}

hipError_t launch_gdn(const GdnArgs& p, float* ws, hipStream_t s) {
  const dim3 prep((unsigned)p.n_chunks, (unsigned)p.hk);
  if (p.in_dtype == NVFP4_DTYPE_BF16)
    gdn_prep_kernel<NVFP4_DTYPE_BF16><<<prep, kPrepThreads, 0, s>>>(p, ws);
  else
    gdn_prep_kernel<NVFP4_DTYPE_F32><<<prep, kPrepThreads, 0, s>>>(p, ws);
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
