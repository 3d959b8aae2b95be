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
//     (I + M) U = R,  R = diag(beta) (V - diag(G) K S0^T),
//     M[t][j] = beta_t (G_t / G_j) k_t.k_j  (j < t),
// so U = T R with T = (I + M)^-1, and
//     O = diag(G) Q S0^T + A U = diag(G) Q S0^T + (A T) R,
//         A[t][j] = (G_t / G_j) q_t.k_j  (j <= t),
//     S_end = G_C S0 + U^T diag(G_C / G) K = G_C S0 + R^T Z,
//         Z = T^T diag(G_C / G) K.
// A T, Z and the per-token factors depend on the chunk only, so one kernel
// computes them for every (key head, chunk) in parallel, sharing k.k^T and
// q.k^T among the value heads of a key head (it never reads v); a second
// walks the chunks in order per (head, 32-row slice of S), forming R from
// its state and the value rows: the rows of S evolve independently, so
// slices need no communication.  The normalized q and k are stored once per
// key head and chunk with G_t per value head, and the scan forms diag(G) Q
// and diag(G) K itself with the same float32 products.
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
constexpr int kScanThreads = 1024;  // scan workgroup: 16 waves
// LDS row strides, padded so the 16 rows a wave reads at once fall into
// distinct banks (an unpadded 512-byte stride puts them all in one)
constexpr int kP = kD + 4;   // rows of 128 floats
constexpr int kPA = kC + 4;  // rows of 64 floats

// Workspace, floats: per (value head, chunk) a block of kWsPerChunk, all
// value heads first; after them per (key head, chunk) a block of
// kWsPerKeyChunk (room is reserved for as many key heads as value heads, so
// the size depends on tokens and value heads only).
constexpr int64_t kWsZ = 0;                  // Z^T = (T^T diag(G_C/G) K)^T  [128][64]
constexpr int64_t kWsAT = kWsZ + kD * kC;    // A T  [64][64]
constexpr int64_t kWsEG = kWsAT + kC * kC;   // G_t = exp(cumulative log decay)  [64]
constexpr int64_t kWsB = kWsEG + kC;         // beta_t  [64]
constexpr int64_t kWsG = kWsB + kC;          // G_C (one float, padded to 4)
constexpr int64_t kWsPerChunk = kWsG + 4;
constexpr int64_t kWsQN = 0;                 // normalized (and 128^-1/2-scaled) q  [64][128]
constexpr int64_t kWsKN = kWsQN + kC * kD;   // normalized k  [64][128]
constexpr int64_t kWsPerKeyChunk = kWsKN + kC * kD;
static_assert(kWsPerChunk % 4 == 0 && kWsPerKeyChunk % 4 == 0, "blocks keep 16-byte alignment");

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

// One workgroup per (chunk, key head), two per CU (69 KB of LDS each), so
// one workgroup's loads, barriers and serial steps overlap the other's
// products.  Everything but the 16x16 diagonal blocks of the triangular
// inverse runs on v_mfma_f32_16x16x4f32.  Inside a product's 16-wide K
// block the lane group g = lane/16 takes k = 4g + s at MFMA step s (any
// order of k gives the same sum): an operand read along k is one 16-byte
// LDS read per 4 steps, a product's accumulator (lane holds D[4g + r][lane%16])
// is directly the B operand of a next product, and the accumulator of
// X Y^T is the A operand of a product with Y X^T on the left.
//   1. k rows, L2-normalized, into LDS; waves 4-7 hold one normalized q row
//      per lane in registers (operand order); both go to the workspace.
//      K K^T (waves 0-3, row block w) and K Q^T (waves 4-7, column block
//      w - 4: rows of Q K^T in A-operand order) stay in registers for every
//      value head.
//   2. per value head: M = (beta_t G_t/G_j k_t.k_j)_{j<t} into LDS and
//      A = (G_t/G_j q_t.k_j)_{j<=t} in registers; T = (I + M)^-1 block by
//      block -- diagonal 16x16 blocks by forward substitution, then
//      T_ij = -T_ii sum_{i>k>=j} M_ik T_kj one block diagonal at a time --
//      and T^T in M's place; Z = T^T diag(G_C/G) K (waves 0-3, 32 key
//      columns each) and A T (waves 4-7, one row block each) out.
// The next head's beta and g are loaded before this head's work.
template <int DT>
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void gdn_prep_kernel(GdnArgs p, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) float sk[kC][kP];    // k rows (normalized)
  __shared__ __attribute__((aligned(16))) float smt[kC][kPA];  // M (strictly lower), then T^T (upper blocks)
  __shared__ __attribute__((aligned(16))) float st[kC][kPA];   // T = (I + M)^-1 (lower blocks)
  __shared__ __attribute__((aligned(16))) float sgam[kC];      // cumulative log decay
  __shared__ __attribute__((aligned(16))) float sbeta[kC];     // beta_j
  __shared__ __attribute__((aligned(16))) float segc[kC];      // G_C / G_t

  const int chunk = blockIdx.x, hk = blockIdx.y;
  const int rep = p.hv / p.hk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int gmat = wave >> 2, rb = wave & 3;  // waves 0-3: K K^T row block rb; 4-7: K Q^T column block rb
  const int64_t t0 = (int64_t)chunk * kC;
  const int rt = tid >> 3, part = tid & 7;  // k rows: row rt, elements 16 part ..
  const bool rvalid = t0 + rt < p.T;
  const int64_t rrow = rvalid ? t0 + rt : p.T - 1;       // clamped, always a valid address
  const int64_t lrow = t0 + lane < p.T ? t0 + lane : p.T - 1;
  float* kout = ws + key_block(p.hv, p.n_chunks, hk, chunk);

  // the first head's beta and g go out with q and k
  float bn = 0.0f, gn = 0.0f;
  auto load_head = [&](int h) {
    bn = load_elem<DT>(p.beta, lrow * p.ld_beta + h);
    gn = load_elem<DT>(p.g, lrow * p.ld_g + h);
  };
  load_head(hk * rep);
  // waves 4-7: q row 16 rb + li, elements 16 m + 4 lg + s (m < 8, s < 4)
  floatx4 qv[8];
  if (gmat) {
    const bool qvalid = t0 + 16 * rb + li < p.T;
    const int64_t qrow = qvalid ? t0 + 16 * rb + li : p.T - 1;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if constexpr (DT == NVFP4_DTYPE_BF16) {
        const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p.q) + qrow * p.ld_q +
                                                         (int64_t)hk * kD + 16 * m + 4 * lg);
        qv[m] = floatx4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                        __uint_as_float(w.y & 0xFFFF0000u)};
      } else {
        qv[m] = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(p.q) + qrow * p.ld_q +
                                                  (int64_t)hk * kD + 16 * m + 4 * lg);
      }
    }
    float iq = qvalid ? 1.0f : 0.0f;  // rows past T are zero
    if (p.normalize) {
      float sq2 = 0.0f;
#pragma unroll
      for (int m = 0; m < 8; ++m) sq2 += qv[m][0] * qv[m][0] + qv[m][1] * qv[m][1] + qv[m][2] * qv[m][2] + qv[m][3] * qv[m][3];
      sq2 += __shfl_xor(sq2, 16);
      sq2 += __shfl_xor(sq2, 32);
      iq *= 0.08838834764831845f / fmaxf(sqrtf(sq2), 1e-30f);  // 128^-1/2 / |q|
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      qv[m] *= iq;
      *reinterpret_cast<floatx4*>(kout + kWsQN + (16 * rb + li) * kD + 16 * m + 4 * lg) = qv[m];
    }
  }
  {
    float kr[16];
    load16<DT>(p.k, rrow * p.ld_k + (int64_t)hk * kD + part * 16, kr);
    float ik = rvalid ? 1.0f : 0.0f;  // rows past T are zero
    if (p.normalize) {
      float sk2 = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) sk2 += kr[e] * kr[e];
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) sk2 += __shfl_xor(sk2, off);
      ik *= 1.0f / fmaxf(sqrtf(sk2), 1e-30f);
    }
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const floatx4 kv = {kr[e] * ik, kr[e + 1] * ik, kr[e + 2] * ik, kr[e + 3] * ik};
      *reinterpret_cast<floatx4*>(&sk[rt][part * 16 + e]) = kv;
      *reinterpret_cast<floatx4*>(kout + kWsKN + rt * kD + part * 16 + e) = kv;
    }
  }
  __syncthreads();

  // waves 0-3: gram[cb][r] = (K K^T)[16 rb + 4 lg + r][16 cb + li];
  // waves 4-7: gram[cb][r] = (K Q^T)[16 cb + 4 lg + r][16 rb + li]
  //                        = (Q K^T)[16 rb + li][16 cb + 4 lg + r]
  floatx4 gram[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) gram[cb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  if (gmat == 0) {
#pragma unroll 2
    for (int k0 = 0; k0 < kD; k0 += 16) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(&sk[16 * rb + li][k0 + 4 * lg]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const floatx4 b = *reinterpret_cast<const floatx4*>(&sk[16 * cb + li][k0 + 4 * lg]);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) gram[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s2], b[s2], gram[cb], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(&sk[16 * cb + li][16 * m + 4 * lg]);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          gram[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s2], qv[m][s2], gram[cb], 0, 0, 0);
      }
    }
  }

  for (int hr = 0; hr < rep; ++hr) {
    const int h = hk * rep + hr;
    float* out = ws + ((int64_t)h * p.n_chunks + chunk) * kWsPerChunk;
    __syncthreads();  // every read of the previous head's smt, st, sgam, sbeta, segc is done
    if (wave == 0) {
      const bool ok = t0 + lane < p.T;  // tokens past T: beta = 0, g = 0
      const float b = ok ? bn : 0.0f;
      const float gam = wave_prefix_sum(ok ? gn : 0.0f, lane);
      sbeta[lane] = b;
      sgam[lane] = gam;
      segc[lane] = expf(__shfl(gam, 63) - gam);
      out[kWsEG + lane] = expf(gam);
      out[kWsB + lane] = b;
    }
    __syncthreads();
    load_head(hr + 1 < rep ? h + 1 : h);  // the next head's beta, g (the last head reloads itself)

    // waves 0-3: M into LDS; waves 4-7: A in registers, areg[cb][s] =
    // A[16 rb + li][16 cb + 4 lg + s] (the A operand of A T, block (rb, cb))
    floatx4 areg[4];
    if (gmat == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * rb + 4 * lg + r;
        const float gt = sgam[t], bt = sbeta[t];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int j = 16 * cb + li;
          smt[t][j] = j < t ? bt * expf(gt - sgam[j]) * gram[cb][r] : 0.0f;
        }
      }
    } else {
      const int t = 16 * rb + li;
      const float gt = sgam[t];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * cb + 4 * lg + r;
          areg[cb][r] = j <= t ? expf(gt - sgam[j]) * gram[cb][r] : 0.0f;
        }
    }
    if (tid == 0) out[kWsG] = expf(sgam[kC - 1]);  // G_C
    __syncthreads();  // M complete

    // diagonal blocks of T: lane (block i, column c) solves (I + M_ii) x = e_c
    if (wave == 0) {
      // the lane's column through an opaque copy: otherwise the sixteen
      // unit-vector constants are kept live across the head loop
      int lane_h;
      asm volatile("v_mov_b32 %0, %1" : "=v"(lane_h) : "v"(lane));
      const int i = lane_h >> 4, c = lane_h & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = r == c ? 1.0f : 0.0f;
#pragma unroll
        for (int jj = 0; jj < r; ++jj) v -= smt[16 * i + r][16 * i + jj] * x[jj];
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
          const floatx4 a = *reinterpret_cast<const floatx4*>(&smt[16 * i + li][16 * kb + 4 * lg]);
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
      __syncthreads();  // (the last one: T complete, every read of M done)
    }
    // T^T in M's place: smt[j][m] = T[m][j] for the lower blocks of T
    // (diagonal blocks whole, zeros above their diagonal included)
    for (int e = tid; e < kC * kC; e += kPrepThreads) {
      const int m = e >> 6, j = e & 63;
      if ((m >> 4) >= (j >> 4)) smt[j][m] = st[m][j];
    }
    __syncthreads();

    if (gmat == 0) {
      // Z = T^T diag(G_C/G) K on key columns 32 rb .. 32 rb + 31, all four
      // token blocks (T^T is upper block-triangular); stored transposed
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int db = 2 * rb + half;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
          for (int jb = tb; jb < 4; ++jb) {
            const floatx4 a = *reinterpret_cast<const floatx4*>(&smt[16 * tb + li][16 * jb + 4 * lg]);
            const floatx4 cf = *reinterpret_cast<const floatx4*>(&segc[16 * jb + 4 * lg]);
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s2], cf[s2] * sk[16 * jb + 4 * lg + s2][16 * db + li], acc,
                                                         0, 0, 0);
          }
          // lane holds Z[16 tb + 4 lg + r][16 db + li], r < 4: four consecutive floats of Z^T
          *reinterpret_cast<floatx4*>(out + kWsZ + (16 * db + li) * kC + 16 * tb + 4 * lg) = acc;
        }
      }
    } else {
      // A T, row block rb: blocks tj <= rb sum A_{rb,mb} T_{mb,tj} over
      // mb = tj..rb; the blocks right of the diagonal are zero
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if (mb < tj || mb > rb) continue;
          const floatx4 b = *reinterpret_cast<const floatx4*>(&smt[16 * tj + li][16 * mb + 4 * lg]);
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(areg[mb][s2], b[s2], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) out[kWsAT + (16 * rb + 4 * lg + r) * kC + 16 * tj + li] = acc[r];
      }
    }
  }
}

// One workgroup (16 waves) per (value head, 32-row slice of S); chunks in
// order.  The three products of a chunk run on v_mfma_f32_16x16x4f32 (fp32
// in, fp32 accumulate; lane l supplies A[l%16][l/16] and B[l/16][l%16] and
// holds D[4(l/16)+r][l%16]); inside each 16-wide K block lane group l/16
// takes k = 4(l/16) + s at step s, so operands are 16-byte LDS reads (R is
// kept transposed, Z arrives transposed).  One 16x16 tile per wave and phase,
// four waves per SIMD to cover each other's operand and barrier latency:
//   phase 1, wave w: tile (t: 16 ti.., c: 16 tj..), ti = (w%8)/2, tj = w%2,
//            of Y = diag(G) K S^T (w < 8; then R = diag(beta) (V - Y)) or
//            of O = diag(G) Q S^T (w >= 8);
//   phase 2, waves w >= 8: O += (A T) R, stored; every wave w: the state
//            tile S[16 (w/8)..][16 (w%8)..] = G_C S + R^T Z.
// The next chunk's data is loaded into registers while one is computed.

constexpr int kKQGroups = kC * kD / 4 / kScanThreads;  // 4-float groups per thread of q, k rows
constexpr int kZGroups = kD * kC / 4 / kScanThreads;   // of Z^T
constexpr int kAGroups = kC * kC / 4 / kScanThreads;   // of A T
static_assert(kKQGroups >= 1 && kZGroups >= 1 && kAGroups >= 1, "every thread loads whole groups");

// A chunk's data in registers, in two halves loaded at different points:
// the normalized k and q rows with G_t (read by the first phase of a step),
// and Z^T, A T, the lane's value elements and beta_t, and G_C (read by the
// second).  Thread tid holds 4-float groups tid + kScanThreads i of each
// array.  Native vector types: arrays of HIP's float4 class stay in scratch
// memory.
__device__ __attribute__((always_inline)) inline void scan_load_kq(const float* in, const float* kin, int tid,
                                                                     floatx4 (&k)[kKQGroups], floatx4 (&q)[kKQGroups],
                                                                     float (&eg)[kKQGroups]) {
#pragma unroll
  for (int i = 0; i < kKQGroups; ++i) {
    const int f = tid + i * kScanThreads;
    k[i] = reinterpret_cast<const floatx4*>(kin + kWsKN)[f];
    q[i] = reinterpret_cast<const floatx4*>(kin + kWsQN)[f];
    eg[i] = in[kWsEG + f / (kD / 4)];  // the row (token) of the group
  }
}
// vrow: the first of the lane's four tokens (rows past T are clamped: their
// beta is 0); vcol: the lane's value column.
template <int DT>
__device__ __attribute__((always_inline)) inline void scan_load_za(const float* in, const GdnArgs& p, int tid,
                                                                     int boff, int64_t vrow, int64_t vcol,
                                                                     floatx4 (&z)[kZGroups], floatx4 (&a)[kAGroups],
                                                                     float (&v)[4], floatx4& beta, float& gc) {
#pragma unroll
  for (int i = 0; i < kZGroups; ++i) z[i] = reinterpret_cast<const floatx4*>(in + kWsZ)[tid + i * kScanThreads];
#pragma unroll
  for (int i = 0; i < kAGroups; ++i) a[i] = reinterpret_cast<const floatx4*>(in + kWsAT)[tid + i * kScanThreads];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = vrow + r < p.T ? vrow + r : p.T - 1;
    v[r] = load_elem<DT>(p.v, row * p.ld_v + vcol);
  }
  beta = *reinterpret_cast<const floatx4*>(in + kWsB + boff);
  gc = in[kWsG];
}

template <int DT, int ODT>
__global__ __launch_bounds__(kScanThreads) void gdn_scan_kernel(GdnArgs p, const float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) float sS[kSlice][kP];  // this slice of the state
  __shared__ __attribute__((aligned(16))) float sK[kC][kP];      // diag(G) K
  __shared__ __attribute__((aligned(16))) float sQ[kC][kP];      // diag(G) Q
  __shared__ __attribute__((aligned(16))) float sZT[kD][kPA];    // Z^T
  __shared__ __attribute__((aligned(16))) float sA[kC][kPA];     // A T
  __shared__ __attribute__((aligned(16))) float sRT[kSlice][kPA];  // R^T: slice rows x tokens

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
  const bool oprod = wave >= 8;                          // phase 1: O tile (else Y tile)
  const int ti = (wave & 7) >> 1, tj = wave & 1;         // the phase-1 tile
  const int tc = wave >> 3, cbk = wave & 7;              // the phase-2 state tile
  const int row0 = sl * kSlice;
  const float* base = ws + (int64_t)h * p.n_chunks * kWsPerChunk;
  const float* kbase = ws + key_block(p.hv, p.n_chunks, h / (p.hv / p.hk), 0);
  const int last = p.n_chunks - 1;

  const int boff = 16 * ti + 4 * lk;                 // the lane's four tokens in a chunk
  const int64_t vcol = (int64_t)h * kD + row0 + 16 * tj + li;  // and its value column
  floatx4 nk[kKQGroups], nq[kKQGroups], nz[kZGroups], na[kAGroups], nb;
  float neg[kKQGroups], nv[4], ngc;

  auto put_kq = [&]() {  // diag(G) K, diag(G) Q registers -> LDS
#pragma unroll
    for (int i = 0; i < kKQGroups; ++i) {
      const int f = tid + i * kScanThreads;
      const int rr = f / (kD / 4), cc = (f % (kD / 4)) * 4;
      *reinterpret_cast<floatx4*>(&sK[rr][cc]) = nk[i] * neg[i];
      *reinterpret_cast<floatx4*>(&sQ[rr][cc]) = nq[i] * neg[i];
    }
  };
  auto put_za = [&]() {  // Z^T, A T registers -> LDS
#pragma unroll
    for (int i = 0; i < kZGroups; ++i) {
      const int f = tid + i * kScanThreads;
      *reinterpret_cast<floatx4*>(&sZT[f / (kC / 4)][(f % (kC / 4)) * 4]) = nz[i];
    }
#pragma unroll
    for (int i = 0; i < kAGroups; ++i) {
      const int f = tid + i * kScanThreads;
      *reinterpret_cast<floatx4*>(&sA[f / (kC / 4)][(f % (kC / 4)) * 4]) = na[i];
    }
  };

  for (int i = tid; i < kSlice * kD; i += kScanThreads) {
    const int c = i / kD, d = i % kD;
    sS[c][d] = p.s0 != nullptr ? p.s0[((int64_t)h * kD + row0 + c) * kD + d] : 0.0f;
  }
  scan_load_kq(base, kbase, tid, nk, nq, neg);
  scan_load_za<DT>(base, p, tid, boff, boff, vcol, nz, na, nv, nb, ngc);
  put_kq();
  __syncthreads();

  // Two barriers per chunk.  Phase 1 reads diag(G) K, diag(G) Q and S;
  // phase 2 reads A T, Z^T, R and writes S.  So Z^T and A T of this chunk go
  // to LDS at the end of phase 1 and the next chunk's diag(G) K, diag(G) Q
  // at the end of phase 2, each half loaded into registers one phase
  // earlier.  Loads are unconditional (the last chunk reloads itself): a
  // load under a branch makes the compiler wait for it where the paths join.
  for (int chunk = 0; chunk < p.n_chunks; ++chunk) {
    const int cn = min(chunk + 1, last);
    const float* nxt = base + (int64_t)cn * kWsPerChunk;
    const float* knxt = kbase + (int64_t)cn * kWsPerKeyChunk;
    // ---- phase 1
    scan_load_kq(nxt, knxt, tid, nk, nq, neg);
    // this wave's tile of Y = diag(G) K S^T or O = diag(G) Q S^T
    floatx4 acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
    {
      const float(*src)[kP] = oprod ? sQ : sK;
#pragma unroll
      for (int kb = 0; kb < kD / 16; ++kb) {
        const floatx4 bs = *reinterpret_cast<const floatx4*>(&sS[16 * tj + li][16 * kb + 4 * lk]);
        const floatx4 as = *reinterpret_cast<const floatx4*>(&src[16 * ti + li][16 * kb + 4 * lk]);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(as[s2], bs[s2], acc1, 0, 0, 0);
      }
    }
    if (!oprod)
      *reinterpret_cast<floatx4*>(&sRT[16 * tj + li][16 * ti + 4 * lk]) =
          floatx4{nb[0] * (nv[0] - acc1[0]), nb[1] * (nv[1] - acc1[1]), nb[2] * (nv[2] - acc1[2]),
                  nb[3] * (nv[3] - acc1[3])};
    put_za();
    __syncthreads();  // R, Z^T, A T of this chunk in LDS; every read of diag(G) K, diag(G) Q, S done
    // ---- phase 2
    const float gc = ngc;
    scan_load_za<DT>(nxt, p, tid, boff, (int64_t)cn * kC + boff, vcol, nz, na, nv, nb, ngc);
    if (oprod) {
      // O += (A T) R over key blocks kb <= ti (A T is lower triangular)
      for (int kb = 0; kb <= ti; ++kb) {
        const floatx4 aa = *reinterpret_cast<const floatx4*>(&sA[16 * ti + li][16 * kb + 4 * lk]);
        const floatx4 br = *reinterpret_cast<const floatx4*>(&sRT[16 * tj + li][16 * kb + 4 * lk]);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(aa[s2], br[s2], acc1, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t tt = (int64_t)chunk * kC + 16 * ti + 4 * lk + q;
        if (tt < p.T) {
          const int64_t idx = tt * p.ld_o + (int64_t)h * kD + row0 + 16 * tj + li;
          if constexpr (ODT == NVFP4_DTYPE_BF16)
            reinterpret_cast<uint16_t*>(p.o)[idx] = (uint16_t)f32_to_bf16_bits(acc1[q]);
          else
            reinterpret_cast<float*>(p.o)[idx] = acc1[q];
        }
      }
    }
    // S[16 tc + i][16 cbk + j] = G_C S + R^T Z: each wave reads and writes
    // only its own tile of the slice
    {
      floatx4 acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = gc * sS[16 * tc + 4 * lk + q][16 * cbk + li];
#pragma unroll
      for (int kb = 0; kb < kC / 16; ++kb) {
        const floatx4 ar = *reinterpret_cast<const floatx4*>(&sRT[16 * tc + li][16 * kb + 4 * lk]);
        const floatx4 bz = *reinterpret_cast<const floatx4*>(&sZT[16 * cbk + li][16 * kb + 4 * lk]);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[s2], bz[s2], acc, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) sS[16 * tc + 4 * lk + q][16 * cbk + li] = acc[q];
    }
    put_kq();         // the next chunk's diag(G) K, diag(G) Q
    __syncthreads();  // new S, next diag(G) K and Q in LDS; every read of this chunk's A T, Z^T, R done
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
  const bool in16 = p.in_dtype == NVFP4_DTYPE_BF16, out16 = p.o_dtype == NVFP4_DTYPE_BF16;
  if (in16 && out16)
    gdn_scan_kernel<NVFP4_DTYPE_BF16, NVFP4_DTYPE_BF16><<<blocks, kScanThreads, 0, s>>>(p, ws);
  else if (in16)
    gdn_scan_kernel<NVFP4_DTYPE_BF16, NVFP4_DTYPE_F32><<<blocks, kScanThreads, 0, s>>>(p, ws);
  else if (out16)
    gdn_scan_kernel<NVFP4_DTYPE_F32, NVFP4_DTYPE_BF16><<<blocks, kScanThreads, 0, s>>>(p, ws);
  else
    gdn_scan_kernel<NVFP4_DTYPE_F32, NVFP4_DTYPE_F32><<<blocks, kScanThreads, 0, s>>>(p, ws);
  return hipGetLastError();
}

}  // namespace nvfp4
