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
//  * cs = (d*sc)[n] * d_a[t], per sub-block: d*sc (at most 17 significant
//    bits) as three pieces sw1..sw3, d_a (11 bits) as two, da1 and da2.  One
//    v_mfma_f32_32x32x8_bf16 whose two K halves hold (sw1 sw2 sw3 0) against
//    (da1 da1 da1 0) and (da2 da2 da2 0) sums the six exact piece products;
//  * the min term (dmin*m)[n] * (d_a*S)[t]: three pieces each (d_a*S has at
//    most 23 bits).  Eight of the nine piece products (the dropped w3*x3 is
//    below 2^-32 of the term) fill the eight K slots of one sub-block, so
//    one v_mfma_f32_32x32x16_bf16 covers two sub-blocks; it accumulates over
//    all of k in its own accumulator, subtracted at the end.
// The vector ALUs then do one conversion and one FMA per output element and
// sub-block: acc += cs * float(P).
//
// Tiling: a workgroup of eight wavefronts computes 128 tokens x 128 weight
// rows (gate/up pass: 64 rows of each matrix).  Each wavefront owns 32
// tokens x 64 weight rows (or 32 tokens x 32 rows of both matrices): two
// 32x32 tiles.  Weight rows are the MFMA A operand (rows), tokens the B
// operand (columns); lane l holds token l%32 and rows 8*(i/4) + 4*(l/32) + i%4.
//
// Staging: per half block (128 k values, four sub-blocks), double-buffered
// in LDS (64 KiB per stage), everything the inner loop reads is already in
// MFMA operand form: the weight quants unpacked to one byte per weight, the
// activation quants (both with a 144-byte row stride, free of bank
// conflicts), and per (row, sub-block) and (token, sub-block) the bfloat16
// scale pieces in the K-slot order of the two scale MFMAs.  The unpacking
// and the scale splitting are done once per workgroup instead of in every
// wavefront that reads them.  Global loads are raw buffer loads (rows past n
// and tokens past m read zeros), issued for half block h+1 before half block
// h is computed.
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
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kBM = 128;                 // tokens per workgroup
constexpr int kWRows = 128;              // staged weight rows per workgroup (both matrices)
constexpr int kThreads = 512;
constexpr int kHalf = kQK / 2;           // k values per stage
constexpr int kSubHalf = kHalf / kSub;   // sub-blocks per stage
constexpr int kRowStride = kHalf + 16;   // LDS row of quants (bytes)

// One LDS stage.  bfloat16 pieces, two per 32-bit word (first K slot in the
// low half):
//   wc [sub-block][row]   (sw1 sw2, sw3 0)               cs, both K halves
//   xc [sub-block][token] (da1 da1, da1 0 | da2 da2, da2 0) cs, K half 0 | 1
//   wm [sub-block][row]   (w1 w1, w1 w2, w2 w2, w3 w3)   min, sw = d*sc,
//   xm [sub-block][token] (x1 x2, x3 x1, x2 x3, x1 x2)   w = dmin*m, x = d_a*S
struct Stage {
  uint8_t w[kWRows * kRowStride];  // unpacked weight quants [row][128]
  uint8_t x[kBM * kRowStride];     // activation quants [token][128]
  uint2 wc[kSubHalf * kWRows];
  uint4 xc[kSubHalf * kBM];
  uint4 wm[kSubHalf * kWRows];
  uint4 xm[kSubHalf * kBM];
};
static_assert(sizeof(Stage) == 65536, "stage layout");

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

// v = p1 + p2 exactly for v with at most 16 significant bits.
__device__ __forceinline__ void split2(float v, uint32_t& p1, uint32_t& p2) {
  p1 = bf16_rne(v);
  p2 = bf16_rne(v - __uint_as_float(p1 << 16));
}

__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0);
}

// Staging registers of one half block for one thread.
struct Loads {
  uint4 wq;     // packed quants: LDS row tid / 4, 16-byte chunk tid % 4 of the half
  uint4 wh;     // block header of LDS row tid % 128
  uint4 xq[2];  // activation quant chunks
  uint32_t xd;  // activation scale word: token tid % 128, sub-block tid / 128 of the half
};

template <bool GU>
struct Geometry {
  // LDS weight row -> (matrix, row within the workgroup's rows)
  __device__ static int row(int lr) { return GU ? (lr & 63) : lr; }
  static constexpr int kRowsPerMatrix = GU ? 64 : 128;
};

// Byte offsets of this thread's staging loads for half block 0 (kOob for
// rows past n, tokens past m, and the activation scales of the partials test
// hook, which passes none); half block hb = 2b + h adds b * 144 + 64h to the
// quants, b * 144 to the header, 128 hb to the activations and 16 hb to the
// scale words.
struct LoadOffsets {
  uint32_t wq, wh, xq[2], xd;
};

// GATHER (grouped gate/up pass): activation row t of the tile is qs/ds row
// group_list[t0 + t] / group_top_k, relative to the whole qs/ds.
template <bool GU, bool PARTIALS, bool GATHER>
__device__ __forceinline__ LoadOffsets load_offsets(const MmqArgs& a, int K, int nsub, int rows,
                                                    int t0, int toks, int tid) {
  LoadOffsets o;
  {
    const int lr = tid >> 2, c = tid & 3;
    const int r = Geometry<GU>::row(lr);
    o.wq = r < rows ? static_cast<uint32_t>(r * K) * kBlockBytes + 16u + 16u * c : kOob;
  }
  {
    const int r = Geometry<GU>::row(tid & 127);
    o.wh = r < rows ? static_cast<uint32_t>(r * K) * kBlockBytes : kOob;
  }
  auto src_row = [&](int t) {
    if constexpr (GATHER) return a.group_list[t0 + t] / a.group_top_k;
    else return t;
  };
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + i * kThreads;
    const int t = idx >> 3, c = idx & 7;
    o.xq[i] = t < toks ? static_cast<uint32_t>(src_row(t)) * a.k + 16u * c : kOob;
  }
  {
    const int t = tid & 127, jj = tid >> 7;
    o.xd = !PARTIALS && t < toks ? (static_cast<uint32_t>(src_row(t)) * nsub + jj) * 4u : kOob;
  }
  return o;
}

// Issues the staging loads of half block hb (all zeros when hb == hend: the
// last iteration's prefetch).  The matrix of every weight load is uniform in
// the wavefront (quant chunks: LDS rows 16w .. 16w+15, i.e. matrix w / 4 of
// the fused pass; headers: rows 64(w%2) .. +63), so the buffer resource is
// picked without a per-lane select (which the compiler would turn into a
// loop over the distinct resources).
template <bool GU, bool PARTIALS>
__device__ __forceinline__ void issue_loads(const LoadOffsets& o, rsrc_t rw0, rsrc_t rw1, rsrc_t rx,
                                            rsrc_t rd, int hend, int hb, int wave, Loads& L) {
  // Uniform deltas; past the end every delta is kDead, which puts each
  // offset (at most kOob plus a real delta) at or above every resource's
  // size without wrapping, so those loads read zeros.
  constexpr uint32_t kDead = 0x40000000u;
  const bool live = hb < hend;
  const uint32_t dw = live ? static_cast<uint32_t>(hb >> 1) * kBlockBytes : kDead;
  const uint32_t dq = live ? dw + static_cast<uint32_t>(hb & 1) * (kHalf / 2) : kDead;
  const uint32_t dx = live ? static_cast<uint32_t>(hb) * kHalf : kDead;
  const uint32_t dd = live ? static_cast<uint32_t>(hb) * (kSubHalf * 4) : kDead;
  L.wq = buf_load16(GU && wave >= 4 ? rw1 : rw0, o.wq + dq);
  L.wh = buf_load16(GU && (wave & 1) ? rw1 : rw0, o.wh + dw);
#pragma unroll
  for (int i = 0; i < 2; ++i) L.xq[i] = buf_load16(rx, o.xq[i] + dx);
  if constexpr (PARTIALS) {
    L.xd = 0u;
  } else {
    L.xd = buf_load4(rd, o.xd + dd);
  }
}

// 6-bit scale and min of sub-block 4H + u of a block header (u uniform,
// 0..3): for the first half, the low 6 bits of scales[u] and scales[u+4];
// for the second, the low and high nibbles of scales[u+8] below the top two
// bits of scales[u] (scale) and scales[u+4] (min).
template <int H>
__device__ __forceinline__ void scale_min_half(const uint4& h, int u, uint32_t& sc, uint32_t& mn) {
  const int sh = 8 * u;
  if constexpr (H == 0) {
    sc = (h.y >> sh) & 63u;
    mn = (h.z >> sh) & 63u;
  } else {
    const uint32_t b1 = h.y >> sh, b2 = h.z >> sh, b3 = h.w >> sh;
    sc = (b3 & 15u) | ((b1 >> 2) & 48u);
    mn = ((b3 >> 4) & 15u) | ((b2 >> 2) & 48u);
  }
}

// Writes the stage of a half block with parity H (quants of bytes 64H ..
// 64H+63 of each block's quant field, sub-blocks 4H .. 4H+3).
template <bool GU, bool PARTIALS, int H>
__device__ __forceinline__ void store_stage(Stage& S, const Loads& L, int wave, int tid) {
  // Quant chunk c of the half's 64 packed bytes: positions 16(c%2) .. +15 of
  // sub-block 2(c/2) (low nibbles) and 2(c/2) + 1 (high nibbles).
  {
    const int lr = tid >> 2, c = tid & 3;
    const int base = lr * kRowStride + 64 * (c >> 1) + 16 * (c & 1);
    const uint4 v = L.wq;
    *reinterpret_cast<uint4*>(&S.w[base]) =
        make_uint4(v.x & 0x0F0F0F0Fu, v.y & 0x0F0F0F0Fu, v.z & 0x0F0F0F0Fu, v.w & 0x0F0F0F0Fu);
    *reinterpret_cast<uint4*>(&S.w[base + kSub]) =
        make_uint4((v.x >> 4) & 0x0F0F0F0Fu, (v.y >> 4) & 0x0F0F0F0Fu, (v.z >> 4) & 0x0F0F0F0Fu,
                   (v.w >> 4) & 0x0F0F0F0Fu);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + i * kThreads;
    const int t = idx >> 3, c = idx & 7;
    *reinterpret_cast<uint4*>(&S.x[t * kRowStride + 16 * c]) = L.xq[i];
  }
  if constexpr (!PARTIALS) {
    const int r = tid & 127, jj = wave >> 1;  // LDS row or token; sub-block of the half (uniform)
    {
      const float d = half_bits_to_float(L.wh.x & 0xFFFFu);
      const float dmin = half_bits_to_float(L.wh.x >> 16);
      uint32_t sc, mn, s1, s2, s3, m1, m2, m3;
      scale_min_half<H>(L.wh, jj, sc, mn);
      split3(d * static_cast<float>(sc), s1, s2, s3);  // exact products
      split3(dmin * static_cast<float>(mn), m1, m2, m3);
      S.wc[jj * kWRows + r] = make_uint2(s1 | (s2 << 16), s3);
      S.wm[jj * kWRows + r] = make_uint4(m1 | (m1 << 16), m1 | (m2 << 16), m2 | (m2 << 16), m3 | (m3 << 16));
    }
    {
      const float da = half_bits_to_float(L.xd & 0xFFFFu);
      const float sa = da * static_cast<float>(static_cast<int16_t>(L.xd >> 16));  // exact
      uint32_t d1, d2, a1, a2, a3;
      split2(da, d1, d2);
      split3(sa, a1, a2, a3);
      S.xc[jj * kBM + r] = make_uint4(d1 | (d1 << 16), d1, d2 | (d2 << 16), d2);
      S.xm[jj * kBM + r] = make_uint4(a1 | (a2 << 16), a3 | (a1 << 16), a2 | (a3 << 16), a1 | (a2 << 16));
    }
  }
}

// GRP: grouped (MoE prefill) pass, the tile from a.group_tiles; GATHER: its
// activation rows gathered through a.group_list (the gate/up pass).
template <bool GU, bool PARTIALS, bool GRP, bool GATHER>
__global__ __launch_bounds__(kThreads) void mmq_kernel(MmqArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Stage* stages = reinterpret_cast<Stage*>(smem);
  constexpr int RPM = Geometry<GU>::kRowsPerMatrix;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // wm 0..3: token tile; wn 0..1: weight half
  const int n0 = (static_cast<int>(blockIdx.x) + a.row_tile0) * RPM;
  const int K = a.k / kQK;
  const int nsub = a.k / kSub;
  const int rows = min(RPM, a.n - n0);
  int t0, toks;
  size_t wofs = static_cast<size_t>(n0) * K * kBlockBytes;
  if constexpr (GRP) {
    // tile g: {expert, first row of the sorted row space, rows}; grid rows
    // past the tile count exit before touching anything
    const int g = blockIdx.y;
    if (g >= *a.group_count) return;
    const int4 td = reinterpret_cast<const int4*>(a.group_tiles)[g];
    t0 = __builtin_amdgcn_readfirstlane(td.y);
    toks = __builtin_amdgcn_readfirstlane(td.z);
    wofs += static_cast<size_t>(__builtin_amdgcn_readfirstlane(td.x)) * a.group_mat_bytes;
  } else {
    t0 = blockIdx.y * kBM;
    toks = min(kBM, a.m - t0);
  }

  // resources: this workgroup's weight rows of each matrix and token rows
  // (a gathering pass addresses all of qs/ds by token row)
  const uint32_t wbytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(K) * kBlockBytes;
  const rsrc_t rw0 = make_rsrc(a.w + wofs, wbytes);
  const rsrc_t rw1 = GU ? make_rsrc(a.w_up + wofs, wbytes) : rw0;
  const size_t xrow0 = GATHER ? 0 : static_cast<size_t>(t0);
  const uint32_t xrows = GATHER ? static_cast<uint32_t>(a.m) : static_cast<uint32_t>(toks);
  const rsrc_t rx = make_rsrc(a.qs + xrow0 * a.k, xrows * a.k);
  // (no activation scales in the partials hook: an empty resource)
  const rsrc_t rd = make_rsrc(a.ds ? a.ds + xrow0 * nsub : a.ds,
                              a.ds && !PARTIALS ? xrows * nsub * 4u : 0u);

  // this lane's operand rows: weight tile wt in {0, 1} -> LDS weight row
  const int r32 = lane & 31;
  const int kh = lane >> 5;  // K half of the MFMA operands
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

  // this workgroup's half blocks: all of k, or split z of a k-split pass
  const int kb0 = blockIdx.z * a.split_blocks;
  const int kb1 = min(K, kb0 + a.split_blocks);
  const int hb0 = 2 * kb0, hb1 = 2 * kb1;

  const LoadOffsets lo = load_offsets<GU, PARTIALS, GATHER>(a, K, nsub, rows, t0, toks, tid);
  // Staging loads run two half blocks ahead of the compute: L0 holds even
  // half blocks, L1 odd ones, and the loop covers one whole block (two half
  // blocks) per iteration so that both register sets keep fixed names.
  // Global latency under load (weights come from HBM or the Infinity Cache)
  // exceeds one half block of compute.
  auto compute = [&](const Stage& S, int hb) {
    __builtin_amdgcn_sched_barrier(0);
    // Units u = 2*jj + wt (sub-block jj of the half, weight tile wt) run as a
    // three-stage software pipeline inside the wavefront: while the VALU
    // converts and scales unit u, the two MFMAs of unit u+1 are in flight and
    // the LDS operands of unit u+2 are being read, so neither the LDS nor
    // the matrix-core latency stalls the wavefront.
    v4i av[2], xv[2];
    v2u32 ca[2], cb[2];
    v16i P[2];
    v16f C[2];
    uint4 mb, ma[2];
    auto load_ops = [&](int u) {
      const int jj = u >> 1, wt = u & 1;
      if (wt == 0) {
        xv[jj & 1] = *reinterpret_cast<const v4i*>(&S.x[xtok * kRowStride + kSub * jj + 16 * kh]);
        if constexpr (!PARTIALS)
          cb[jj & 1] =
              *reinterpret_cast<const v2u32*>(reinterpret_cast<const uint8_t*>(&S.xc[jj * kBM + xtok]) + 8 * kh);
      }
      av[u & 1] = *reinterpret_cast<const v4i*>(&S.w[wrow[wt] * kRowStride + kSub * jj + 16 * kh]);
      if constexpr (!PARTIALS) {
        const uint2 c = S.wc[jj * kWRows + wrow[wt]];
        ca[u & 1] = v2u32{c.x, c.y};
      }
    };
    auto issue = [&](int u) {
      const int jj = u >> 1;
      P[u & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[u & 1], xv[jj & 1], zi, 0, 0, 0);
      if constexpr (!PARTIALS)
        C[u & 1] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(v4s, ca[u & 1]),
                                                             __builtin_bit_cast(v4s, cb[jj & 1]), zf, 0, 0, 0);
    };
    // min term: K half kh of MFMA i2 is sub-block 2*i2 + kh
    auto load_min = [&](int i2) {
      mb = S.xm[(2 * i2 + kh) * kBM + xtok];
#pragma unroll
      for (int wt = 0; wt < 2; ++wt) ma[wt] = S.wm[(2 * i2 + kh) * kWRows + wrow[wt]];
    };
    auto min_term = [&]() {
#pragma unroll
      for (int wt = 0; wt < 2; ++wt)
        accm[wt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ma[wt]),
                                                            __builtin_bit_cast(v8bf, mb), accm[wt], 0, 0, 0);
    };
    constexpr int kUnits = 2 * kSubHalf;
    load_ops(0);
    load_ops(1);
    issue(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int jj = u >> 1, wt = u & 1;
      const v16i Pu = P[u & 1];
      const v16f Cu = C[u & 1];
      if (u + 1 < kUnits) issue(u + 1);
      if constexpr (!PARTIALS) {
        if (u == 2 || u == 6) min_term();
      }
      if (u + 2 < kUnits) load_ops(u + 2);
      if constexpr (!PARTIALS) {
        if (u == 0 || u == 4) load_min(u / 4);
      }
      if constexpr (PARTIALS) {
        // fence: the scheduler keeps each pipeline step in this order
        __builtin_amdgcn_sched_barrier(0);
        // C row i of this lane: weight row 8*(i/4) + 4*kh + i%4 of the tile
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int lr = (GU ? wt * 64 + wn * 32 : wn * 64 + wt * 32) + 8 * (i >> 2) + 4 * kh + (i & 3);
          const int r = Geometry<GU>::row(lr);
          if (r < rows && xtok < toks)
            a.partials[(static_cast<size_t>(t0 + xtok) * a.n + n0 + r) * nsub + kSubHalf * hb + jj] = Pu[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[wt][i] = fmaf(Cu[i], static_cast<float>(Pu[i]), acc[wt][i]);
        // The step's MFMAs (unit u+1, min term) and LDS reads (unit u+2) do
        // not depend on its VALU work (unit u): spread them through it, so a
        // wavefront issues them while the SIMD's VALU runs the other
        // wavefront's instructions instead of both stalling the VALU at once.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  Loads L0, L1;
  issue_loads<GU, PARTIALS>(lo, rw0, rw1, rx, rd, hb1, hb0, wave, L0);
  store_stage<GU, PARTIALS, 0>(stages[0], L0, wave, tid);
  issue_loads<GU, PARTIALS>(lo, rw0, rw1, rx, rd, hb1, hb0 + 1, wave, L1);
  issue_loads<GU, PARTIALS>(lo, rw0, rw1, rx, rd, hb1, hb0 + 2, wave, L0);
  __syncthreads();

  for (int hb = hb0; hb < hb1; hb += 2) {
    // stage 1 was last read in the previous iteration, before its closing
    // barrier; stage 0 in the first half of this one
    compute(stages[0], hb);
    store_stage<GU, PARTIALS, 1>(stages[1], L1, wave, tid);
    issue_loads<GU, PARTIALS>(lo, rw0, rw1, rx, rd, hb1, hb + 3, wave, L1);
    __syncthreads();
    compute(stages[1], hb + 1);
    store_stage<GU, PARTIALS, 0>(stages[0], L0, wave, tid);
    issue_loads<GU, PARTIALS>(lo, rw0, rw1, rx, rd, hb1, hb + 4, wave, L0);
    __syncthreads();
  }

  if constexpr (GU && !PARTIALS) {
    if (a.gu_parts != nullptr) {  // uniform: a k split of the fused pass
      // gate and up sums of this split, rows wn*32 + 8*(i/4) + 4*kh + i%4
      if (xtok < toks) {
        const size_t ld = static_cast<size_t>(a.row_tiles) * RPM;
        const size_t tok = static_cast<size_t>(t0 + xtok);
        const size_t r0 = static_cast<size_t>(n0 - a.row_tile0 * RPM);
        float* pg = a.gu_parts + (static_cast<size_t>(2 * blockIdx.z) * a.m + tok) * ld + r0;
        float* pu = pg + static_cast<size_t>(a.m) * ld;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = wn * 32 + 8 * (i >> 2) + 4 * kh + (i & 3);
          if (r < rows) {
            pg[r] = acc[0][i] - accm[0][i];
            pu[r] = acc[1][i] - accm[1][i];
          }
        }
      }
    } else if (a.q_out != nullptr) {  // uniform
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
      const int orow = GRP && a.group_scatter ? a.group_list[t0 + xtok] : t0 + xtok;
      const size_t roff = blockIdx.z * a.split_stride + static_cast<size_t>(orow) * a.n;
      if constexpr (GU) {
        if (a.q_out == nullptr && a.gu_parts == nullptr) {
          float* yrow = a.y + roff;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = wn * 32 + 8 * (i >> 2) + 4 * kh + (i & 3);
            if (r < rows) yrow[n0 + r] = silu_mul(acc[0][i] - accm[0][i], acc[1][i] - accm[1][i]);
          }
        }
      } else if (a.y_bf16 != nullptr) {
        // the result stored as bfloat16 straight from the tile
        uint16_t* brow = a.y_bf16 + roff;
#pragma unroll
        for (int wt = 0; wt < 2; ++wt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = wn * 64 + wt * 32 + 8 * (i >> 2) + 4 * kh + (i & 3);
            if (r < rows) brow[n0 + r] = static_cast<uint16_t>(float_to_bf16_rne(acc[wt][i] - accm[wt][i]));
          }
      } else {
        float* yrow = a.y + roff;
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

template <bool GU, bool PARTIALS, bool GRP = false, bool GATHER = false>
hipError_t launch(const MmqArgs& a, hipStream_t stream) {
  constexpr int RPM = Geometry<GU>::kRowsPerMatrix;
  const dim3 grid(a.row_tiles > 0 ? a.row_tiles : (a.n + RPM - 1) / RPM,
                  GRP ? a.group_grid_rows : (a.m + kBM - 1) / kBM, a.splits);
  const size_t lds = 2 * sizeof(Stage);
  auto kern = mmq_kernel<GU, PARTIALS, GRP, GATHER>;
  const hipError_t e = lds_opt_in(reinterpret_cast<const void*>(kern), lds);
  if (e != hipSuccess) return e;
  kern<<<grid, dim3(kThreads), lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mmq(const MmqArgs& args, hipStream_t stream) {
  MmqArgs a = args;
  const int K = a.k / kQK;
  if (a.q_out && (!a.w_up || !a.d_out || a.partials || a.n % 64)) return hipErrorInvalidValue;
  if (a.y_bf16 && (a.w_up || a.partials || a.splits > 1)) return hipErrorInvalidValue;
  // a range of row tiles: dense passes only, inside the matrix
  if (a.row_tiles != 0 || a.row_tile0 != 0) {
    const int rpm = a.w_up ? 64 : 128;
    if (a.group_tiles || a.partials || a.row_tiles < 1 || a.row_tile0 < 0 ||
        a.row_tile0 + a.row_tiles > (a.n + rpm - 1) / rpm)
      return hipErrorInvalidValue;
  }
  // k-split sums of the fused pass: over a range of row tiles, no epilogue
  if (a.gu_parts && (!a.w_up || a.q_out || a.row_tiles < 1)) return hipErrorInvalidValue;
  if (a.splits <= 1 || (a.w_up && !a.gu_parts) || a.partials) {
    a.splits = 1;
    a.split_blocks = K;
    a.split_stride = 0;
  } else if (a.split_blocks < 1 || static_cast<long long>(a.splits - 1) * a.split_blocks >= K) {
    return hipErrorInvalidValue;  // every split must own at least one block
  }
  if (a.group_tiles) {
    // grouped passes: the fused gate/up pass gathers token rows and writes
    // Q8_1(h) in sorted order; the down pass reads those rows and scatters
    if (!a.group_count || !a.group_list || a.partials || a.y_bf16 || a.group_grid_rows < 1)
      return hipErrorInvalidValue;
    if (a.w_up) {
      if (!a.q_out || a.group_top_k < 1 || a.group_scatter) return hipErrorInvalidValue;
      return launch<true, false, true, true>(a, stream);
    }
    if (a.group_top_k != 0) return hipErrorInvalidValue;
    return launch<false, false, true, false>(a, stream);
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

// One 32-lane half of a wavefront per (token, 32-row block of h).
__global__ __launch_bounds__(256) void gu_finish_kernel(const float* __restrict__ parts, int splits, int m,
                                                        int rows, int row0, int n, int8_t* __restrict__ q_out,
                                                        uint32_t* __restrict__ d_out) {
  const int blk = static_cast<int>(blockIdx.x) * 8 + static_cast<int>(threadIdx.x >> 5);
  const int nblk = rows / 32;
  if (blk >= m * nblk) return;  // uniform in the half wavefront
  const int t = blk / nblk;
  const int r = (blk - t * nblk) * 32 + static_cast<int>(threadIdx.x & 31);
  const size_t plane = static_cast<size_t>(m) * rows;
  const size_t at = static_cast<size_t>(t) * rows + r;
  float g = 0.f, u = 0.f;
  for (int z = 0; z < splits; ++z) {
    g += parts[2 * z * plane + at];
    u += parts[(2 * z + 1) * plane + at];
  }
  const float hv = silu_mul(g, u);
  float amax = fabsf(hv);
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
  const float d = q8_1_scale(amax);
  const int q = q8_1_quant(hv, amax, d);
  int sum = q;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 32);
  const size_t row = static_cast<size_t>(row0) + r;
  q_out[static_cast<size_t>(t) * n + row] = static_cast<int8_t>(q);
  if ((threadIdx.x & 31) == 0) d_out[static_cast<size_t>(t) * (n / 32) + row / 32] = q8_1_word(amax, d, sum);
}

}  // namespace

hipError_t launch_mmq_gu_finish(const float* parts, int splits, int m, int rows, int row0, int n,
                                int8_t* q_out, uint32_t* d_out, hipStream_t stream) {
  if (splits < 1 || m < 1 || rows < 32 || rows % 32 || row0 % 32 || n % 32 || row0 + rows > n)
    return hipErrorInvalidValue;
  const long long blocks = (static_cast<long long>(m) * (rows / 32) + 7) / 8;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  gu_finish_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(parts, splits, m, rows, row0, n,
                                                                                   q_out, d_out);
  return hipGetLastError();
}

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
