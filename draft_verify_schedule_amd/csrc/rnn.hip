// RNN head of the sequential draft stage (DSpark paper, section 3.1, RNN
// head; "Speculative decoding, from zero to DSpark", section 6).
//
// The head keeps a state s_k in R^r per request.  At position k it forms
// z_k = [s_{k-1}; W1[x_{k-1}]; h_k] (s_0 = 0) and applies one projection W
// whose 3r rows are the gate, candidate and output parts.  The page's update
// equation did not survive; the reading taken is a GRU-style blend with no
// additive bias:
//   g = sigmoid(W_g z),  c~ = tanh(W_c z),  o = W_o z,  s_k = (1 - g) s_{k-1} + g c~.
// o_k is the bias input in front of W2: the draft stages it where the Markov
// head has W1[x_{k-1}].
//
// Launches:
//   rnn_hproj  once per draft: the hidden-state part W[:, 2r:] h_k of every
//              (request, position), an MFMA GEMM (B*K x d) x (d x 3r); h does
//              not depend on the sampled tokens, so this leaves the
//              sequential loop;
//   rnn_step   once per position: the state and embedding parts on MFMA (the
//              fp32 state split into three bf16 operands), then the gates;
//   w2_to_f16  once per call: the fp16 copy of W2 that the output parts
//              (staged as hi + lo fp16) meet in the draft's bias MFMA.
#include <algorithm>

#include "bias_tile.hpp"
#include "launch.hpp"
#include "rnn.hpp"

namespace dspark {

// ---------------------------------------------------------------- hproj --
// 128 x 128 output tile per workgroup (n: projection rows, m: (request,
// position) rows) and one slice of the contraction (blockIdx.y of hp_split:
// the 32-column stages are dealt in contiguous ranges), so that the
// full-size GEMM (168 tiles) gives every CU about three workgroups (40 KB of
// LDS each): the kernel is bound by the latency of each stage's loads, which
// the other workgroups of the CU hide.
// 4 waves in 2 x 2, each 64 x 64 = 4 x 4 MFMA blocks with A = W rows (n) and
// B = h rows (m): lane l ends with 4 consecutive n of one m, stored as one
// 16-byte vector into the slice's partial.  The stages run through
// double-buffered LDS; rows past M or N read as zero through the buffer
// resources' range check.
constexpr int kHpTile = 128;
constexpr int kHpK = 32;
constexpr int kHpPitch = kHpK + 8;  // bf16 per LDS row: 80 bytes
constexpr int kHpChunks = kHpTile * kHpK / 8 / 256;  // 16-byte chunks per thread and operand

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void rnn_hproj_kernel(RnnParams p, int mtiles,
                                                                                            int ntiles) {
  int mt, nt;
  if (!xcd_tile(blockIdx.x, mtiles, ntiles, mt, nt)) return;
  __shared__ uint16_t hs[2][kHpTile][kHpPitch];
  __shared__ uint16_t ws[2][kHpTile][kHpPitch];
  const int M = p.B * p.K, N = 3 * p.r, d = p.d;
  const int ldw = 2 * p.r + d;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int wn = wave >> 1, wm = wave & 1;
  const int m0 = mt * kHpTile, n0 = nt * kHpTile;
  const int nk_all = p.d / kHpK;
  const int kt0 = (int)((int64_t)blockIdx.y * nk_all / p.hp_split);
  const int kt1 = (int)((int64_t)(blockIdx.y + 1) * nk_all / p.hp_split);
  float* const out = p.Hp + (size_t)blockIdx.y * M * N;
  const uint32_t hbytes = (uint32_t)((uint64_t)M * d * 2);
  const uint32_t wbytes = (uint32_t)((uint64_t)N * ldw * 2);
  const rsrc_t hr = make_rsrc(p.H, hbytes);
  const rsrc_t wr = make_rsrc(p.W, wbytes);
  // global -> LDS: kHpChunks 16-byte chunks per thread and operand; chunk
  // id / (kHpK / 8) is the tile row, id % (kHpK / 8) the 8-column group
  uint32_t hoff[kHpChunks], woff[kHpChunks];
  int lrow[kHpChunks], lcol[kHpChunks];
#pragma unroll
  for (int q = 0; q < kHpChunks; ++q) {
    const int id = tid + 256 * q;
    lrow[q] = id / (kHpK / 8);
    lcol[q] = (id % (kHpK / 8)) * 8;
    const int m = m0 + lrow[q], n = n0 + lrow[q];
    hoff[q] = m < M ? (uint32_t)(((uint64_t)m * d + lcol[q]) * 2) : hbytes;
    woff[q] = n < N ? (uint32_t)(((uint64_t)n * ldw + 2 * p.r + lcol[q]) * 2) : wbytes;
  }
  u32x4 hv[kHpChunks], wv[kHpChunks];
  auto gload = [&](int kt) {
    const uint32_t so = (uint32_t)kt * (kHpK * 2);
#pragma unroll
    for (int q = 0; q < kHpChunks; ++q) {
      hv[q] = buffer_load16(hr, hoff[q], so);
      wv[q] = buffer_load16(wr, woff[q], so);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kHpChunks; ++q) {
      *reinterpret_cast<u32x4*>(&hs[buf][lrow[q]][lcol[q]]) = hv[q];
      *reinterpret_cast<u32x4*>(&ws[buf][lrow[q]][lcol[q]]) = wv[q];
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nk = kt1 - kt0;  // at least one stage: hp_split <= d / 64
  gload(kt0);
  lstore(0);
  __syncthreads();
  const int fr = lane & 15, fk = 8 * (lane >> 4);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt0 + kt + 1);
#pragma unroll
    for (int kc = 0; kc < kHpK / 32; ++kc) {
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(&ws[buf][64 * wn + 16 * i + fr][32 * kc + fk]);
        bf[i] = *reinterpret_cast<const bf16x8*>(&hs[buf][64 * wm + 16 * i + fr][32 * kc + fk]);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[nb], bf[mb], acc[nb][mb], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + 64 * wn + 16 * nb + 4 * (lane >> 4);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + 64 * wm + 16 * mb + fr;
      if (m < M && n < N) *reinterpret_cast<f32x4*>(out + (size_t)m * N + n) = acc[nb][mb];
    }
  }
}

// ----------------------------------------------------------------- step --
// One workgroup per (16 state units j, 16 requests).  MFMA A operands are W
// rows (gate, candidate, output row of unit j), B operands the z rows of the
// requests, so lane l ends with units j0 + 4 (l / 16) + i of request
// b0 + l % 16.  The four waves split the contraction by 32-column chunk
// (chunk c on wave c % 4): state chunks as three bf16 terms (together the
// fp32 value), embedding chunks as the bf16 W1 row itself.  Their partial sums meet in LDS in wave
// order; wave 0 adds the hidden-state part and applies the gates.
__global__ __launch_bounds__(256) void rnn_step_kernel(RnnParams p, int k, const float* __restrict__ s_prev,
                                                       float* __restrict__ s_next) {
  const int r = p.r, ldw = 2 * r + p.d;
  const int jtiles = r / 16;
  const int jt = blockIdx.x % jtiles, bt = blockIdx.x / jtiles;
  const int j0 = 16 * jt, b0 = 16 * bt;
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int b = b0 + (lane & 15);
  const bool b_ok = b < p.B;
  const int kq = 8 * (lane >> 4);
  int prev = -1;
  if (b_ok) prev = k == 1 ? p.x0[b] : p.x[(size_t)b * p.K + k - 2];
  const bool e_ok = prev >= 0 && prev < p.V;
  const uint16_t* wrow[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) wrow[c] = p.W + (size_t)(c * r + j0 + (lane & 15)) * ldw;
  f32x4 acc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nch = r / 32;
  if (s_prev) {  // s_0 = 0 adds nothing
    for (int c = wave; c < nch; c += 4) {
      const int kk = 32 * c + kq;
      f32x4 v0 = f32x4{0.f, 0.f, 0.f, 0.f}, v1 = v0;
      if (b_ok) {
        v0 = *reinterpret_cast<const f32x4*>(s_prev + (size_t)b * r + kk);
        v1 = *reinterpret_cast<const f32x4*>(s_prev + (size_t)b * r + kk + 4);
      }
      // s = t0 + t1 + t2 in bf16 terms, each the rounded remainder of the
      // previous: 24 significant bits, the fp32 state itself
      u32x4 t[3];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float f0 = e < 2 ? v0[2 * e] : v1[2 * e - 4];
        float f1 = e < 2 ? v0[2 * e + 1] : v1[2 * e - 3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const uint32_t h0 = bf16_rne_bits(f0), h1 = bf16_rne_bits(f1);
          t[q][e] = h0 | (h1 << 16);
          f0 -= __uint_as_float(h0 << 16);
          f1 -= __uint_as_float(h1 << 16);
        }
      }
#pragma unroll
      for (int comp = 0; comp < 3; ++comp) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(wrow[comp] + kk);
#pragma unroll
        for (int q = 0; q < 3; ++q)
          acc[comp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, t[q]), acc[comp], 0, 0, 0);
      }
    }
  }
  for (int c = wave; c < nch; c += 4) {
    const int kk = 32 * c + kq;
    const u32x4 ev = e_ok ? *reinterpret_cast<const u32x4*>(p.W1 + (size_t)prev * r + kk) : u32x4{0u, 0u, 0u, 0u};
    const bf16x8 z = __builtin_bit_cast(bf16x8, ev);
#pragma unroll
    for (int comp = 0; comp < 3; ++comp) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(wrow[comp] + r + kk);
      acc[comp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, z, acc[comp], 0, 0, 0);
    }
  }
  __shared__ f32x4 red[4][3][64];
#pragma unroll
  for (int comp = 0; comp < 3; ++comp) red[wave][comp][lane] = acc[comp];
  __syncthreads();
  if (wave != 0 || !b_ok) return;
  f32x4 pre[3];
#pragma unroll
  for (int comp = 0; comp < 3; ++comp)
    pre[comp] = ((red[0][comp][lane] + red[1][comp][lane]) + red[2][comp][lane]) + red[3][comp][lane];
  const int jj = j0 + 4 * (lane >> 4);
  const size_t row = (size_t)b * p.K + (k - 1);
  // the hidden-state part: the projection's slice partials added in order
  f32x4 hg = f32x4{0.f, 0.f, 0.f, 0.f}, hc = hg, ho = hg;
  const size_t slice = (size_t)p.B * p.K * 3 * r;
  for (int q = 0; q < p.hp_split; ++q) {
    const float* hp = p.Hp + q * slice + row * (size_t)(3 * r);
    hg += *reinterpret_cast<const f32x4*>(hp + jj);
    hc += *reinterpret_cast<const f32x4*>(hp + r + jj);
    ho += *reinterpret_cast<const f32x4*>(hp + 2 * r + jj);
  }
  f32x4 sp = f32x4{0.f, 0.f, 0.f, 0.f};
  if (s_prev) sp = *reinterpret_cast<const f32x4*>(s_prev + (size_t)b * r + jj);
  f32x4 sn, o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float g = 1.f / (1.f + expf(-(pre[0][i] + hg[i])));
    const float cand = tanhf(pre[1][i] + hc[i]);
    sn[i] = (1.f - g) * sp[i] + g * cand;
    o[i] = pre[2][i] + ho[i];
  }
  *reinterpret_cast<f32x4*>(s_next + (size_t)b * r + jj) = sn;
  *reinterpret_cast<f32x4*>(p.O + row * r + jj) = o;
}

// ------------------------------------------------------------ W2 to fp16 --
// bf16 -> fp32 is exact; fp32 -> fp16 rounds to nearest even, exact for every
// bf16 of magnitude 2^-14 .. 2^15 (8 significant bits fit in 11), with at
// most 2^-25 absolute error below that range.
// ------------------------------------------------------------------ host --
static size_t align256_rnn(size_t n) { return (n + 255) / 256 * 256; }

int run_w2_swizzle(const uint16_t* W2, void* out, int V, int r, int kc, bool f16, hipStream_t stream);

// The RNN head's kernels run with eight k chunks for every r (zero-padded),
// so its fp16 fragment-ordered copy holds eight chunks per block.
constexpr int kRnnChunks = 8;
size_t w2_f16_bytes(int V, int r) {
  (void)r;
  return (size_t)(((int64_t)V + 63) / 64) * 4 * kRnnChunks * 1024;
}

// Contraction slices of the projection GEMM: enough (tile, slice) workgroups
// for about three per CU, at most 4, never more than the d / 32 stages.
static int rnn_hp_split(int B, int K, int r, int d) {
  const int tiles = ((B * K + kHpTile - 1) / kHpTile) * ((3 * r + kHpTile - 1) / kHpTile);
  return std::max(1, std::min({4, 768 / tiles, d / kHpK}));
}

size_t rnn_workspace_bytes(int B, int K, int V, int r, int d, bool with_w2h) {
  return align256_rnn((size_t)rnn_hp_split(B, K, r, d) * B * K * 3 * r * sizeof(float)) +
         2 * align256_rnn((size_t)B * r * sizeof(float)) + (with_w2h ? w2_f16_bytes(V, r) : 0);
}

void rnn_bind_workspace(RnnParams& p, void* workspace) {
  char* ws = reinterpret_cast<char*>(workspace);
  p.hp_split = rnn_hp_split(p.B, p.K, p.r, p.d);
  p.Hp = reinterpret_cast<float*>(ws);
  ws += align256_rnn((size_t)p.hp_split * p.B * p.K * 3 * p.r * sizeof(float));
  p.s[0] = reinterpret_cast<float*>(ws);
  ws += align256_rnn((size_t)p.B * p.r * sizeof(float));
  p.s[1] = reinterpret_cast<float*>(ws);
  ws += align256_rnn((size_t)p.B * p.r * sizeof(float));
  if (!p.w2h_ready) p.W2h = reinterpret_cast<uint16_t*>(ws);
}

int run_w2_to_f16(const uint16_t* W2, uint16_t* out, int V, int r, hipStream_t stream) {
  return run_w2_swizzle(W2, out, V, r, kRnnChunks, true, stream);
}

int run_rnn_hproj(const RnnParams& p, hipStream_t stream) {
  const int mtiles = (p.B * p.K + kHpTile - 1) / kHpTile;
  const int ntiles = (3 * p.r + kHpTile - 1) / kHpTile;
  return launch_kernel("rnn_hproj", rnn_hproj_kernel, dim3(xcd_grid(mtiles, ntiles), p.hp_split), dim3(256), stream,
                       p, mtiles, ntiles);
}

int run_rnn_step(const RnnParams& p, int k, hipStream_t stream) {
  const float* s_prev = k == 1 ? nullptr : p.s[(k - 1) & 1];
  float* s_next = p.s[k & 1];
  const int grid = (p.r / 16) * ((p.B + 15) / 16);
  return launch_kernel("rnn_step", rnn_step_kernel, dim3(grid), dim3(256), stream, p, k, s_prev, s_next);
}

}  // namespace dspark
