// Streaming small-M (decode) FP8 block-scaled NT GEMM for gfx950.
//
// Same operation as the tiled kernel (FP8 block-quantised GEMM page on
// lpnh.cn, s2.2 and s3.2; NT layout per the DeepGEMM page on pzsr.cn, s3.1)
// for M <= 64, where the time is the stream of B (N x K bytes) from HBM.
//
// gfx950 mapping
//  * Every wave streams its own strip of RW rows of B (RW = 16, 32 or 64) over
//    its own share of K, with direct global loads that land already in the
//    v_mfma_f32_16x16x128_f8f6f4 fragment layout (lane l holds row l%16 and
//    32 K bytes chosen by l/16).  Loads are double-buffered in registers, U K
//    blocks per buffer, so 2*U*RW*128 bytes per wave are in flight and no LDS
//    or barrier sits in the main loop; with several waves per SIMD this keeps
//    enough bytes in flight per CU to stream B at HBM speed.
//  * A workgroup's 4 waves cover 4/KS strips; the KS waves of a strip split
//    its K range (KS = 1 when K is short, 4 when N is small) and add their FP32
//    accumulators through LDS in wave order at the end (deterministic).
//  * The main loop has no branches (divergent or uniform): lanes for A rows
//    >= M re-read row 0 and get a zero scale, and K blocks past a wave's range
//    re-read its last block with a zero scale; branches around the loads make
//    the compiler wait for every outstanding load at each merge.
//  * Each 128-K partial is promoted with sa(m,kb)*sb(n,kb) in FP32; outputs
//    are rounded to BF16 once.
#include "dg_device.hpp"
#include "dg_internal.hpp"

#include <stdlib.h>

namespace dg {
namespace {

constexpr int BK = 128;

struct StreamArgs {
  uint16_t* c;
  Epilogue epi;
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  const uint32_t* sfa;  // E8: packed UE8M0 exponents (four K blocks per word)
  const uint32_t* sfb;
  int a_block_rows;
  int M, N, K;
  int nkb;
  int sa_stride;  // ceil(M / a_block_rows)
  int sb_stride;  // ceil(N / 128)
};

// E8: power-of-two (UE8M0) scales (DeepGEMM page on pzsr.cn, s3.1) applied
// by the scaled MFMA, accumulators chained through K.  UE8M0 has no zero, so
// K blocks past a wave's range zero their B fragment instead of the scale.
template <int RW, int MP, int KS, int U, bool E8 = false>
__global__ void __launch_bounds__(256) gemm_stream_kernel(StreamArgs p) {
  constexpr int NF = RW / 16;  // B fragments per wave
  constexpr int NI = MP / 16;  // A fragments
  constexpr int SPW = 4 / KS;  // strips per workgroup
  __shared__ float red[KS > 1 ? 4 : 1][NF][NI][4][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int fr = lane & 15;
  const int g = lane >> 4;
  const int strip = blockIdx.x * SPW + wave / KS;
  const int kpart = wave % KS;
  const int n0 = strip * RW;
  // past the last strip (KS == 1 only: no barrier follows); with KS > 1 such
  // waves run on clamped rows and store nothing
  if (KS == 1 && n0 >= p.N) return;

  // this wave's K blocks [kb_begin, kb_end)
  const int kb_begin = (int)((int64_t)kpart * p.nkb / KS);
  const int kb_end = (int)((int64_t)(kpart + 1) * p.nkb / KS);

  const uint8_t* bp[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int row = n0 + 16 * f + fr;
    row = row < p.N ? row : p.N - 1;  // rows past N feed only unstored outputs
    bp[f] = p.b + (int64_t)row * p.K + g * 32;
  }
  const uint8_t* ap[NI];
  float aval[NI];  // 1 for real A rows, 0 for padding rows (their products are dropped)
  int sa_col[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int m = 16 * i + fr;
    const bool real = m < p.M;
    aval[i] = real ? 1.0f : 0.0f;
    ap[i] = p.a + (int64_t)(real ? m : 0) * p.K + g * 32;
    sa_col[i] = p.a_block_rows == 1 ? (real ? m : 0) : 0;
  }
  const int nb = n0 / 128;  // RW divides 128: the strip lies in one B scale block

  struct Buf {
    v8i b[U][NF];
    v8i a[U][NI];
    float sa[U][NI];
    float sb[U];
    int ea[U][NI];  // E8: exponent bytes
    int eb[U];
  };

  // K blocks past this wave's range re-load its last block with a zero scale
  auto load = [&](Buf& x, int kb_first) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = kb_first + u < kb_end;
      const int kb = in ? kb_first + u : kb_end - 1;
      const int64_t ko = (int64_t)kb * BK;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const v4i lo = *reinterpret_cast<const v4i*>(bp[f] + ko);
        const v4i hi = *reinterpret_cast<const v4i*>(bp[f] + ko + 16);
        x.b[u][f] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (E8) x.b[u][f] &= (in ? -1 : 0);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const v4i lo = *reinterpret_cast<const v4i*>(ap[i] + ko);
        const v4i hi = *reinterpret_cast<const v4i*>(ap[i] + ko + 16);
        x.a[u][i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (E8)
          x.ea[u][i] = (int)((p.sfa[(int64_t)(kb >> 2) * p.sa_stride + sa_col[i]] >>
                              (8 * (kb & 3))) & 0xFFu);
        else
          x.sa[u][i] = p.sa[(int64_t)kb * p.sa_stride + sa_col[i]] * aval[i];
      }
      if constexpr (E8) {
        x.eb[u] = (int)((p.sfb[(int64_t)(kb >> 2) * p.sb_stride + nb] >> (8 * (kb & 3))) & 0xFFu);
      } else {
        const float sbv = p.sb[(int64_t)kb * p.sb_stride + nb];
        x.sb[u] = in ? sbv : 0.0f;
      }
    }
  };

  v4f acc[NF][NI];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[f][i] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Buf& x) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          if constexpr (E8) {
            acc[f][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                x.b[u][f], x.a[u][i], acc[f][i], 0, 0, 0, x.eb[u], 0, x.ea[u][i]);
          } else {
            const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                x.b[u][f], x.a[u][i], zero, 0, 0, 0, 0, 0, 0);
            acc[f][i] += part * (x.sa[u][i] * x.sb[u]);
          }
        }
  };

  if (kb_begin < kb_end) {  // uniform per wave; false only when W > K/128
    Buf x0, x1;
    load(x0, kb_begin);
    for (int kb = kb_begin; kb < kb_end; kb += 2 * U) {
      load(x1, kb + U);  // next buffer in flight while x0 is used
      compute(x0);
      load(x0, kb + 2 * U);
      compute(x1);
    }
  }

  // lane owns C[m = 16i + l%16][n = n0 + 16f + 4*(l/16) + r]
  auto store = [&](auto act, auto res, int f, int i, const float* t) {
    const int m = 16 * i + fr;
    const int n = n0 + 16 * f + 4 * g;
    if (m < p.M && n < p.N) store4<decltype(act)::value, decltype(res)::value != 0>(p.c, m, n, t, p.epi);
  };
  if (KS == 1) {
    with_epilogue(p.epi, [&](auto act, auto res) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const float t[4] = {acc[f][i][0], acc[f][i][1], acc[f][i][2], acc[f][i][3]};
          store(act, res, f, i, t);
        }
    });
    return;
  }
  // KS > 1: the workgroup is one strip (SPW == 1 needs KS == 4; KS == 2 gives
  // two strips) -- add the KS partial sums of each strip in wave order
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][f][i][r][lane] = acc[f][i][r];
  __syncthreads();
  if (kpart != 0) return;
  with_epilogue(p.epi, [&](auto act, auto res) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float t[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          t[r] = red[wave][f][i][r][lane];
#pragma unroll
          for (int w = 1; w < KS; ++w) t[r] += red[wave + w][f][i][r][lane];
        }
        store(act, res, f, i, t);
      }
  });
}

template <int RW, int MP, int KS, int U>
hipError_t launch(const StreamArgs& p, hipStream_t stream) {
  constexpr int SPW = 4 / KS;
  const int strips = (p.N + RW - 1) / RW;
  const unsigned grid = (unsigned)((strips + SPW - 1) / SPW);
  if (p.sfa)
    hipLaunchKernelGGL((gemm_stream_kernel<RW, MP, KS, U, true>), dim3(grid), dim3(256), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<RW, MP, KS, U>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Waves per strip: split K across the workgroup's 4 waves only when the strips
// alone give too few waves to keep HBM busy (~1500 waves fill the GPU).
int choose_ks(int64_t strips, int64_t nkb) {
  static const int forced = [] {
    const char* e = getenv("DG_STREAM_KS");
    return e ? atoi(e) : 0;
  }();
  if (forced == 1 || forced == 2 || forced == 4) return forced;
  if (strips >= 1024 || nkb < 8) return 1;
  if (strips >= 384 || nkb < 16) return 2;
  return 4;
}

template <int RW, int MP, int U>
hipError_t launch_ks(const StreamArgs& p, hipStream_t stream) {
  const int ks = choose_ks((p.N + RW - 1) / RW, p.nkb);
  if (ks == 1) return launch<RW, MP, 1, U>(p, stream);
  if (ks == 2) return launch<RW, MP, 2, U>(p, stream);
  return launch<RW, MP, 4, U>(p, stream);
}

}  // namespace

// Measured on MI355X: for M <= 8 the streaming kernel wins unless N alone
// supplies enough 128-row LDS-ring workgroups (N >= 16384).  At M = 16 every
// streaming wave re-reads as many bytes of A as of B, so the ring kernel (A
// staged once per workgroup, split-K) wins once B is large (7168 x 16384),
// while the streaming kernel keeps small B (4096 x 4096).  An override
// DG_DECODE_KERNEL=ring|stream is read once, for tuning sweeps.
bool stream_preferred(int64_t M, int64_t N, int64_t K) {
  static const int forced = [] {
    const char* e = getenv("DG_DECODE_KERNEL");
    return e ? (e[0] == 's' ? 1 : (e[0] == 'r' ? 2 : 0)) : 0;
  }();
  if (forced) return forced == 1;
  return N < 16384 && (M <= 8 || (M <= 16 && N * K <= (int64_t(32) << 20)));
}

hipError_t launch_gemm_stream(const GemmProblem& q, hipStream_t stream) {
  StreamArgs p;
  p.c = q.c; p.a = q.a; p.b = q.b; p.sa = q.sa; p.sb = q.sb;
  p.sfa = q.sfa; p.sfb = q.sfb;
  p.epi = resolved_epilogue(q);
  p.a_block_rows = q.a_block_rows;
  p.M = (int)q.M; p.N = (int)q.N; p.K = (int)q.K;
  p.nkb = (int)(q.K / BK);
  p.sa_stride = (int)((q.M + q.a_block_rows - 1) / q.a_block_rows);
  p.sb_stride = (int)((q.N + 127) / 128);
  if (q.M <= 16) return launch_ks<16, 16, 2>(p, stream);
  if (q.M <= 32) return launch_ks<32, 32, 2>(p, stream);
  return launch_ks<64, 64, 1>(p, stream);
}

}  // namespace dg
