// Q8_1 x Q4_K integer GEMM (MMQ) for the prefill regime, gfx950 int8 MFMA.
//
// "spark_model/layers/ops/q4k_mmq.rs", q4k_mmq_gemm: C[m,n] = A_q8[m,k] x
// W_q4k[n,k]^T; "realizar -- ffn.rs", fused_ffn_swiglu_gpu_true_dp4a: the
// integer dot comes first and the scales are applied afterwards.  For token
// t, weight row n and 32-value sub-block j:
//   P = sum_{i<32} q_w * q_a                          (v_mfma_i32_32x32x32_i8)
//   y += (d*sc_j)[n] * d_a[t,j] * P  -  (dmin*m_j)[n] * (d_a*S)[t,j]
// where S is the integer block sum stored with the activation scale.  One
// 32x32x32 MFMA covers exactly one sub-block, so its int32 result is the
// per-sub-block partial P (the test hook writes it out unchanged).
//
// Both scale products are outer products of a weight-row vector and a token
// vector, so they run on the matrix cores too, on exact bfloat16 pieces with
// f32 accumulation (bfloat16 keeps the f32 exponent range, so saturated or
// tiny scales are carried exactly):
//  * cs = (d*sc)[n] * d_a[t]: d*sc (at most 17 significant bits) as three
//    pieces, d_a (11 bits) as two: 6 K slots of v_mfma_f32_32x32x8_bf16;
//  * the min term (dmin*m)[n] * (d_a*S)[t]: three pieces each (d_a*S has at
//    most 23 bits), 9 K slots of v_mfma_f32_32x32x16_bf16, accumulated over
//    all sub-blocks in its own accumulator and subtracted at the end.
// The vector ALUs then do one conversion and one FMA per output element and
// sub-block: acc += cs * float(P).
//
// Tiling: a workgroup of eight wavefronts computes 128 tokens x 128 weight
// rows (gate/up pass: 64 rows of each matrix).  Each wavefront owns 32
// tokens x 64 weight rows (or 32 tokens x 32 rows of both matrices): two
// 32x32 tiles.  Weight rows are the MFMA A operand (rows), tokens the B
// operand (columns); lane l holds token l%32 and rows 8*(i/4) + 4*(l/32) + i%4.
// Per 256-wide k block the workgroup stages, double-buffered in LDS, the raw
// 144-byte weight blocks (their row stride keeps the fragment reads free of
// bank conflicts), the 128 x 256 activation quants (row stride 272 bytes),
// and per (row, sub-block) and (token, sub-block) the bfloat16 scale pieces.
// Global loads are raw buffer loads (rows past n and tokens past m read
// zeros), issued for block b+1 before block b is computed.
//
// Epilogue modes: y (f32); for the fused gate/up pass either h = silu(g) * u
// or, for the FFN, h quantised to Q8_1 on the spot (lanes l and l+32 hold one
// 32-value block of a token, so its max and sum take one cross-half shuffle
// each); for the single-matrix pass, optionally a split of the k blocks over
// grid z, each split writing its own partial plane (added in order by
// split_reduce_kernel), which fills the device when the row x token tiles
// alone would leave compute units idle.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"
#include "q8_1_device.hpp"

namespace q4k {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v8u32h __attribute__((ext_vector_type(4)));  // eight bfloat16 as four words

constexpr int kBM = 128;          // tokens per workgroup
constexpr int kWRows = 128;       // staged weight rows per workgroup (both matrices)
constexpr int kThreads = 512;
constexpr int kXStride = kQK + 16;  // LDS row of activation quants (bytes)

// One LDS stage.  Scale records are three 32-bit words of bfloat16 pieces,
// stored sub-block-major ([j][row], [j][token]: a 3-word stride between
// lanes, free of bank conflicts):
//   weights (row, sub-block): (sw1, sw2), (sw3, mw1), (mw2, mw3) for
//     sw = d*sc and mw = dmin*m;
//   tokens (token, sub-block): (da1, da2), (sa1, sa2), (sa3, 0) for d_a and
//     sa = d_a*S.
struct Stage {
  uint8_t w[kWRows * kBlockBytes];  // raw blocks, row stride 144
  uint32_t ws[kWRows * 8 * 3];
  uint8_t x[kBM * kXStride];        // activation quants, row stride 272
  uint32_t xs[kBM * 8 * 3];
};

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)));
}

// v = p1 + p2 + p3 exactly (bfloat16 pieces; v has at most 24 significant
// bits, so each residual is exact in binary32).
__device__ __forceinline__ void split3(float v, uint32_t& p1, uint32_t& p2, uint32_t& p3) {
  p1 = bf16_rne(v);
  float r = v - __uint_as_float(p1 << 16);
  p2 = bf16_rne(r);
  r -= __uint_as_float(p2 << 16);
  p3 = bf16_rne(r);
}

// Staging registers of one k block for one thread.
struct Loads {
  uint4 wq[2];   // weight quant chunks
  uint4 wh;      // weight header of row tid % 128
  uint4 xq[4];   // activation quant chunks
  uint2 xd;      // activation scale words: token tid % 128, sub-blocks 2*(tid/128) .. +1
};

template <bool GU>
struct Geometry {
  // LDS weight row -> (matrix, row within the workgroup's rows)
  __device__ static int matrix(int lr) { return GU ? lr >> 6 : 0; }
  __device__ static int row(int lr) { return GU ? (lr & 63) : lr; }
  static constexpr int kRowsPerMatrix = GU ? 64 : 128;
};

// Byte offsets of this thread's staging loads for block 0 (kOob for rows
// past n, tokens past m, and the activation scales of the partials test hook,
// which passes none); block b adds b * 144, b * 256 and b * 32.
struct LoadOffsets {
  uint32_t wq[2], wh, xq[4], xd;
};

template <bool GU, bool PARTIALS>
__device__ __forceinline__ LoadOffsets load_offsets(const MmqArgs& a, int K, int nsub, int rows,
                                                    int toks, int tid) {
  LoadOffsets o;
  // weight quants: 128 rows x 8 chunks of 16 bytes; chunk c of row lr at
  // byte 16 + 16c of the block
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + i * kThreads;
    const int lr = idx >> 3, c = idx & 7;
    const int r = Geometry<GU>::row(lr);
    o.wq[i] = r < rows ? static_cast<uint32_t>(r * K) * kBlockBytes + 16u + 16u * c : kOob;
  }
  {
    const int r = Geometry<GU>::row(tid & 127);
    o.wh = r < rows ? static_cast<uint32_t>(r * K) * kBlockBytes : kOob;
  }
  // activation quants: 128 tokens x 16 chunks of 16 bytes
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + i * kThreads;
    const int t = idx >> 4, c = idx & 15;
    o.xq[i] = t < toks ? static_cast<uint32_t>(t) * a.k + 16u * c : kOob;
  }
  {
    const int t = tid & 127, h = tid >> 7;
    o.xd = !PARTIALS && t < toks ? (static_cast<uint32_t>(t) * nsub + 2 * h) * 4u : kOob;
  }
  return o;
}

// Issues the staging loads of block b (all zeros when b == kend: the last
// iteration's prefetch).
// The matrix of every staging load is uniform in the wavefront (weight chunk
// load i serves LDS rows 64i .. 64i+63, i.e. matrix i of the fused pass; the
// header load of wavefront w serves rows 64(w%2) .. +63), so the buffer
// resource is picked without a per-lane select (which the compiler would
// turn into a loop over the distinct resources).
template <bool GU, bool PARTIALS>
__device__ __forceinline__ void issue_loads(const LoadOffsets& o, rsrc_t rw0, rsrc_t rw1, rsrc_t rx,
                                            rsrc_t rd, int kend, int b, int wave, Loads& L) {
  const bool live = b < kend;  // uniform
  const uint32_t dw = static_cast<uint32_t>(b) * kBlockBytes;
  const uint32_t dx = static_cast<uint32_t>(b) * kQK;
  const uint32_t dd = static_cast<uint32_t>(b) * 32u;
#pragma unroll
  for (int i = 0; i < 2; ++i) L.wq[i] = buf_load16(GU && i == 1 ? rw1 : rw0, live ? o.wq[i] + dw : kOob);
  L.wh = buf_load16(GU && (wave & 1) ? rw1 : rw0, live ? o.wh + dw : kOob);
#pragma unroll
  for (int i = 0; i < 4; ++i) L.xq[i] = buf_load16(rx, live ? o.xq[i] + dx : kOob);
  if constexpr (PARTIALS) {
    L.xd = make_uint2(0u, 0u);
  } else {
    L.xd = buf_load8(rd, live ? o.xd + dd : kOob);
  }
}

template <bool GU, bool PARTIALS>
__device__ __forceinline__ void store_stage(Stage& S, const Loads& L, int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + i * kThreads;
    const int lr = idx >> 3, c = idx & 7;
    *reinterpret_cast<uint4*>(&S.w[lr * kBlockBytes + 16 + 16 * c]) = L.wq[i];
  }
  // weight scales: row tid % 128, sub-blocks 2*(tid/128) .. +1
  {
    const int lr = tid & 127, h = tid >> 7;
    const float d = half_bits_to_float(L.wh.x & 0xFFFFu);
    const float dmin = half_bits_to_float(L.wh.x >> 16);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * h + jj;
      uint32_t sc, mn, s1, s2, s3, m1, m2, m3;
      scale_min_rt(L.wh, j, sc, mn);
      split3(d * static_cast<float>(sc), s1, s2, s3);     // exact product
      split3(dmin * static_cast<float>(mn), m1, m2, m3);
      uint32_t* rec = &S.ws[(j * kWRows + lr) * 3];
      rec[0] = s1 | (s2 << 16);
      rec[1] = s3 | (m1 << 16);
      rec[2] = m2 | (m3 << 16);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + i * kThreads;
    const int t = idx >> 4, c = idx & 15;
    *reinterpret_cast<uint4*>(&S.x[t * kXStride + 16 * c]) = L.xq[i];
  }
  if constexpr (!PARTIALS) {
    const int t = tid & 127, h = tid >> 7;
    const uint32_t wd[2] = {L.xd.x, L.xd.y};
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const float da = half_bits_to_float(wd[jj] & 0xFFFFu);
      const float sa = da * static_cast<float>(static_cast<int16_t>(wd[jj] >> 16));  // exact
      uint32_t d1, d2, d3, a1, a2, a3;
      split3(da, d1, d2, d3);  // d3 = 0: d_a has 11 significant bits
      split3(sa, a1, a2, a3);
      uint32_t* rec = &S.xs[((2 * h + jj) * kBM + t) * 3];
      rec[0] = d1 | (d2 << 16);
      rec[1] = a1 | (a2 << 16);
      rec[2] = a3;
    }
  }
}

template <bool GU, bool PARTIALS>
__global__ __launch_bounds__(kThreads) void mmq_kernel(MmqArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Stage* stages = reinterpret_cast<Stage*>(smem);
  constexpr int RPM = Geometry<GU>::kRowsPerMatrix;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // wm 0..3: token tile; wn 0..1: weight half
  const int t0 = blockIdx.y * kBM;
  const int n0 = blockIdx.x * RPM;
  const int K = a.k / kQK;
  const int nsub = a.k / kSub;
  const int rows = min(RPM, a.n - n0);
  const int toks = min(kBM, a.m - t0);

  // resources: this workgroup's weight rows of each matrix and token rows
  const size_t wofs = static_cast<size_t>(n0) * K * kBlockBytes;
  const uint32_t wbytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(K) * kBlockBytes;
  const rsrc_t rw0 = make_rsrc(a.w + wofs, wbytes);
  const rsrc_t rw1 = GU ? make_rsrc(a.w_up + wofs, wbytes) : rw0;
  const rsrc_t rx = make_rsrc(a.qs + static_cast<size_t>(t0) * a.k, static_cast<uint32_t>(toks) * a.k);
  // (no activation scales in the partials hook: an empty resource)
  const rsrc_t rd = make_rsrc(a.ds ? a.ds + static_cast<size_t>(t0) * nsub : a.ds,
                              a.ds && !PARTIALS ? static_cast<uint32_t>(toks) * nsub * 4u : 0u);

  // this lane's operand rows: weight tile wt in {0, 1} -> LDS weight row
  const int r32 = lane & 31;
  const int kh = lane >> 5;  // K half of the 32-wide operands / slot half of the K=8 ones
  // v_perm selectors (bytes 0-3: second source, 4-7: first source, 0x0C: 0)
  // that build this lane's half of the scale operands from the records
  struct {
    uint32_t c0, c1, m0, m1, m2, m3, b0, b1, b2, b3;
  } sel;
  if (kh == 0) {
    sel = {0x01000100u, 0x03020302u,                              // (sw1 sw1) (sw2 sw2)
           0x03020302u, 0x05040302u, 0x05040504u, 0x07060706u,    // (mw1 mw1) (mw1 mw2) (mw2 mw2) (mw3 mw3)
           0x03020100u, 0x01000504u, 0x05040302u, 0x03020100u};   // (sa1 sa2) (sa3 sa1) (sa2 sa3) (sa1 sa2)
  } else {
    sel = {0x05040504u, 0x0C0C0C0Cu,                              // (sw3 sw3) (0 0)
           0x0C0C0706u, 0x0C0C0C0Cu, 0x0C0C0C0Cu, 0x0C0C0C0Cu,    // (mw3 0) 0 0 0
           0x0C0C0504u, 0x0C0C0C0Cu, 0x0C0C0C0Cu, 0x0C0C0C0Cu};   // (sa3 0) 0 0 0
  }
  const uint32_t lo_mask = kh == 0 ? 0xFFFFFFFFu : 0u;  // cs token slots 2, 3 live in the first half
  int wrow[2];
#pragma unroll
  for (int wt = 0; wt < 2; ++wt) wrow[wt] = GU ? wt * 64 + wn * 32 + r32 : wn * 64 + wt * 32 + r32;
  const int xtok = wm * 32 + r32;

  v16f acc[2], accm[2];
#pragma unroll
  for (int wt = 0; wt < 2; ++wt)
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc[wt][i] = 0.f; accm[wt][i] = 0.f; }
  v16i zi;
#pragma unroll
  for (int i = 0; i < 16; ++i) zi[i] = 0;
  v16f zf;
#pragma unroll
  for (int i = 0; i < 16; ++i) zf[i] = 0.f;

  // this workgroup's k blocks: all of them, or split z of a k-split pass
  const int kb0 = blockIdx.z * a.split_blocks;
  const int kb1 = min(K, kb0 + a.split_blocks);

  const LoadOffsets lo = load_offsets<GU, PARTIALS>(a, K, nsub, rows, toks, tid);
  Loads L;
  issue_loads<GU, PARTIALS>(lo, rw0, rw1, rx, rd, kb1, kb0, wave, L);
  store_stage<GU, PARTIALS>(stages[0], L, tid);
  __syncthreads();

  for (int b = kb0; b < kb1; ++b) {
    // loads of the next block (zeros past the last one) fly during compute
    issue_loads<GU, PARTIALS>(lo, rw0, rw1, rx, rd, kb1, b + 1, wave, L);
    const Stage& S = stages[(b - kb0) & 1];
#pragma unroll 1
    for (int p = 0; p < 4; ++p) {
      // weight fragments of sub-blocks 2p (low nibbles) and 2p+1 (high)
      v4i wq[2];
#pragma unroll
      for (int wt = 0; wt < 2; ++wt)
        wq[wt] = *reinterpret_cast<const v4i*>(&S.w[wrow[wt] * kBlockBytes + 16 + 32 * p + 16 * kh]);
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const int j = 2 * p + hs;
        const v4i xv = *reinterpret_cast<const v4i*>(&S.x[xtok * kXStride + 32 * j + 16 * kh]);
        // scale operands: lanes 0..31 hold the first half of the K slots,
        // lanes 32..63 the second; v_perm with per-lane selectors builds
        // both halves without branches.
        // token side: cs slots [da1 da2 da1 da2 | da1 da2 0 0],
        // min slots [sa1 sa2 sa3 sa1 sa2 sa3 sa1 sa2 | sa3 0 ...]
        v4u32 csb;
        v8u32h mnb;
        {
          const uint32_t* rec = &S.xs[(j * kBM + xtok) * 3];
          const uint32_t x0 = rec[0], x1 = rec[1], x2 = rec[2];
          csb = v4u32{x0, x0 & lo_mask, 0u, 0u};
          mnb = v8u32h{__builtin_amdgcn_perm(x2, x1, sel.b0), __builtin_amdgcn_perm(x2, x1, sel.b1),
                       __builtin_amdgcn_perm(x2, x1, sel.b2), __builtin_amdgcn_perm(x2, x1, sel.b3)};
        }
#pragma unroll
        for (int wt = 0; wt < 2; ++wt) {
          const v4i av = hs == 0 ? (wq[wt] & 0x0F0F0F0F) : ((wq[wt] >> 4) & 0x0F0F0F0F);
          const v16i P = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, xv, zi, 0, 0, 0);
          if constexpr (PARTIALS) {
            // C row i of this lane: weight row 8*(i/4) + 4*kh + i%4 of the tile
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int lr = (GU ? wt * 64 + wn * 32 : wn * 64 + wt * 32) + 8 * (i >> 2) + 4 * kh + (i & 3);
              const int r = Geometry<GU>::row(lr);
              if (r < rows && xtok < toks)
                a.partials[(static_cast<size_t>(t0 + xtok) * a.n + n0 + r) * nsub + b * 8 + j] = P[i];
            }
          } else {
            // weight side: cs slots [sw1 sw1 sw2 sw2 | sw3 sw3 0 0],
            // min slots [mw1 mw1 mw1 mw2 mw2 mw2 mw3 mw3 | mw3 0 ...]
            const uint32_t* rec = &S.ws[(j * kWRows + wrow[wt]) * 3];
            const uint32_t w0 = rec[0], w1 = rec[1], w2 = rec[2];
            const v2u32 csa = v2u32{__builtin_amdgcn_perm(w1, w0, sel.c0), __builtin_amdgcn_perm(w1, w0, sel.c1)};
            const v4u32 mna = v4u32{__builtin_amdgcn_perm(w2, w1, sel.m0), __builtin_amdgcn_perm(w2, w1, sel.m1),
                                    __builtin_amdgcn_perm(w2, w1, sel.m2), __builtin_amdgcn_perm(w2, w1, sel.m3)};
            const v16f cs = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(v4s, csa),
                                                                      __builtin_bit_cast(v4s, v2u32{csb[0], csb[1]}),
                                                                      zf, 0, 0, 0);
            accm[wt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, mna),
                                                                __builtin_bit_cast(v8bf, mnb), accm[wt], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[wt][i] = fmaf(cs[i], static_cast<float>(P[i]), acc[wt][i]);
          }
        }
      }
    }
    // the other stage was last read in the previous iteration, before its
    // closing barrier
    store_stage<GU, PARTIALS>(stages[(b + 1 - kb0) & 1], L, tid);
    __syncthreads();
  }

  if constexpr (GU && !PARTIALS) {
    if (a.q_out != nullptr) {  // uniform
      // Lanes l and l + 32 hold rows wn*32 + 8*(i/4) + 4*kh + i%4 of token
      // xtok: together the 32 values of one Q8_1 block of h (n0 + wn*32 is a
      // multiple of 32 and every row exists, n % 64 == 0).
      float hv[16];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        hv[i] = silu_mul(acc[0][i] - accm[0][i], acc[1][i] - accm[1][i]);
        amax = fmaxf(amax, fabsf(hv[i]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const float d = q8_1_scale(amax);
      int q[16];
      int s = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        q[i] = q8_1_quant(hv[i], amax, d);
        s += q[i];
      }
      s += __shfl_xor(s, 32, 64);
      if (xtok < toks) {
        const size_t tok = static_cast<size_t>(t0 + xtok);
        uint32_t* qrow = reinterpret_cast<uint32_t*>(a.q_out + tok * a.n + n0 + wn * 32);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          qrow[2 * g4 + kh] = pack_q4(q[4 * g4], q[4 * g4 + 1], q[4 * g4 + 2], q[4 * g4 + 3]);
        if (kh == 0) a.d_out[tok * (a.n / 32) + (n0 + wn * 32) / 32] = q8_1_word(amax, d, s);
      }
    }
  }
  if constexpr (!PARTIALS) {
    // lane holds token xtok and, per tile, rows 8*(i/4) + 4*kh + i%4
    if (xtok < toks) {
      float* yrow = a.y + blockIdx.z * a.split_stride + static_cast<size_t>(t0 + xtok) * a.n;
      if constexpr (GU) {
        if (a.q_out == nullptr) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = wn * 32 + 8 * (i >> 2) + 4 * kh + (i & 3);
            if (r < rows) yrow[n0 + r] = silu_mul(acc[0][i] - accm[0][i], acc[1][i] - accm[1][i]);
          }
        }
      } else {
#pragma unroll
        for (int wt = 0; wt < 2; ++wt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = wn * 64 + wt * 32 + 8 * (i >> 2) + 4 * kh + (i & 3);
            if (r < rows) yrow[n0 + r] = acc[wt][i] - accm[wt][i];
          }
      }
    }
  }
}

template <bool GU, bool PARTIALS>
hipError_t launch(const MmqArgs& a, hipStream_t stream) {
  constexpr int RPM = Geometry<GU>::kRowsPerMatrix;
  const dim3 grid((a.n + RPM - 1) / RPM, (a.m + kBM - 1) / kBM, a.splits);
  const size_t lds = 2 * sizeof(Stage);
  auto kern = mmq_kernel<GU, PARTIALS>;
  static bool big_lds = false;  // the opt-in is per kernel and stays set
  if (!big_lds) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
    big_lds = true;
  }
  kern<<<grid, dim3(kThreads), lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mmq(const MmqArgs& args, hipStream_t stream) {
  MmqArgs a = args;
  const int K = a.k / kQK;
  if (a.q_out && (!a.w_up || !a.d_out || a.partials || a.n % 64)) return hipErrorInvalidValue;
  if (a.splits <= 1 || a.w_up || a.partials) {
    a.splits = 1;
    a.split_blocks = K;
    a.split_stride = 0;
  } else if (a.split_blocks < 1 || static_cast<long long>(a.splits - 1) * a.split_blocks >= K) {
    return hipErrorInvalidValue;  // every split must own at least one block
  }
  if (a.partials) return a.w_up ? launch<true, true>(a, stream) : launch<false, true>(a, stream);
  return a.w_up ? launch<true, false>(a, stream) : launch<false, false>(a, stream);
}

int mmq_choose_splits(int m, int n, int k, int max_splits, int cus) {
  const long long tiles = static_cast<long long>((n + kWRows - 1) / kWRows) * ((m + kBM - 1) / kBM);
  const int K = k / kQK;
  int best = 1;
  long long best_cost = -1;
  for (int s = 1; s <= max_splits && s <= K; ++s) {
    const int per = (K + s - 1) / s;
    if ((s - 1) * per >= K) continue;  // an empty split
    const long long rounds = (tiles * s + cus - 1) / cus;
    const long long cost = rounds * per;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

namespace {

__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ parts, int splits,
                                                           size_t stride, size_t count4,
                                                           float* __restrict__ y) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count4) return;
  const float4* p = reinterpret_cast<const float4*>(parts) + i;
  const size_t s4 = stride / 4;
  float4 acc = p[0];
  for (int z = 1; z < splits; ++z) {
    const float4 v = p[z * s4];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  reinterpret_cast<float4*>(y)[i] = acc;
}

}  // namespace

hipError_t launch_mmq_split_reduce(const float* parts, int splits, size_t stride, size_t count,
                                   float* y, hipStream_t stream) {
  if (splits < 1 || count % 4 || stride % 4 || (splits > 1 && stride < count)) return hipErrorInvalidValue;
  const size_t count4 = count / 4;
  if (count4 == 0) return hipSuccess;
  const size_t blocks = (count4 + 255) / 256;
  if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
  split_reduce_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(parts, splits, stride,
                                                                                     count4, y);
  return hipGetLastError();
}

}  // namespace q4k
