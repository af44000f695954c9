// Dequant-fused Q4_K GEMV on the matrix cores (2..8 tokens), gfx950.
//
// "realizar -- q4k_gemv_cached_uses.rs", q4k_gemv_cached_async: y = W x with
// W in block_q4_K [n][k/256] and f32 x of length k; "realizar -- ffn.rs",
// fused_ffn_swiglu_gpu: gate and up GEMVs, silu(gate) * up, then the down
// GEMV.  Here the gate and up GEMVs run in one pass over both matrices and
// the silu * mul is applied before the single store.
//
// The dot products run on the matrix cores (v_mfma_f32_16x16x32_f16) with
// exact operands:
//  * weights: for sub-block j the product sc_j * q is an integer <= 945,
//    exact in binary16, so each 256-block is one chain of 8 K=32 steps whose
//    f32 sum is multiplied by d once; the min term sum_j m_j * X_j (X_j the
//    activation sum of sub-block j) is a second chain over the same
//    activation operand with m_j (<= 63, exact) as the weight operand, its
//    sum multiplied by dmin;
//  * activations: per token and chunk of blocks, x is scaled by 2^sh (sh
//    chosen so the chunk maximum lands in [2^14, 2^15)) and split into two
//    binary16 halves: hi = x rounded toward zero, lo = (x - hi) rounded
//    toward zero (x - hi is exact in f32), together 21 significant bits or
//    more.  The 16 rows of the activation operand hold the hi halves of
//    tokens 0..7 (rows 0..7) and the lo halves (rows 8..15), so one MFMA per
//    step multiplies both halves of every token by the same weight operand;
//    the two result rows of a token are added at the end.
// The relative error of a row result is thus a few 2^-21 of ||w|| ||x||.
//
// Work decomposition: a workgroup (W = 4 or 8 wavefronts) owns RT tiles of
// 16 output rows; the k/256 blocks are split into W contiguous ranges, one
// per wavefront.
// Lane l holds weight row n0 + l%16 and the 64 weights 64*(l/16) .. +63 of
// each block (32 contiguous quant bytes, two 16-byte loads), i.e. the K
// index 8*(l/16)+i of step s is weight 64*(l/16) + 8*s + i; the activation
// operand uses the same K mapping.  Each wavefront converts its own
// activation range a chunk of blocks at a time into LDS in operand layout.
// Split mode (the down pass of the FFN, at most 256 row tiles): every row
// group runs as two workgroups over the two halves of the blocks, which add
// their sums to a y the gate/up pass has zeroed (each workgroup converts the
// activations of half of k instead of all of it); 0 + a + b rounds the same
// in either order, so the result is deterministic.
// Every global load is a raw buffer load (out-of-range lanes read zero); the
// weights of the next tile (or of the next chunk's first tile) and the next
// chunk's activations are in flight while the current ones are multiplied,
// and reductions across lanes use DPP.  The W partial tiles are added in a
// fixed order at the end (deterministic).
#include <type_traits>

#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kWavesMax = 8;  // wavefronts per workgroup: 4, or 8 when the workgroups fit the CUs
constexpr int kRows = 16;  // output rows per workgroup (MFMA N)

// Tokens per half of the activation operand (4 or 8), and blocks converted
// per LDS round.  Two blocks per chunk: a wavefront often owns only two blocks
// of k (k = 4096 over 8 wavefronts), and a larger chunk then loads zeros for
// the rest; one block per chunk leaves too little in flight.
template <int MT> constexpr int half_rows() { return MT <= 4 ? 4 : 8; }
template <int MT> constexpr int chunk_blocks() { return 2; }

// LDS of one wavefront's activation operands for a chunk, R2 = 2 * half_rows:
//   op: [CH][8 steps][4 lane groups][R2 rows] x 8 halves (16 B per entry);
//       rows 0..HR-1 hold the hi halves of the tokens, rows HR..R2-1 the lo
//   shift: [8] exponent sh per token (one per chunk)
// The step stride is padded by one entry (4 R2 + 1) so that one token's
// 8-byte conversion writes (all steps and lane groups at once) spread over the
// banks; with a stride of 4 R2 entries, a multiple of 256 bytes, all eight
// steps hit the same banks (counters: 60-80% of the LDS cycles were bank
// conflicts, 1-7% with the pad; at eight tokens, padding the lane-group
// stride as well, by one or two entries, left 60-80%).  A step's operand
// reads stay one contiguous run per lane group.
template <int MT>
struct WaveLds {
  static constexpr int kCH = chunk_blocks<MT>();
  static constexpr int kR2 = 2 * half_rows<MT>();
  static constexpr int kSG = kR2;          // lane-group stride (entries)
  static constexpr int kSS = 4 * kSG + 1;  // step stride (entries)
  uint4 op[kCH * 8 * kSS];
  int shift[8];
  __device__ static int idx(int bi, int s, int g, int row) { return (bi * 8 + s) * kSS + g * kSG + row; }
};

template <int MT, bool GU, int W>
struct Lds {
  union {
    WaveLds<MT> wave[W];
    float red[GU ? 2 : 1][W][16][kRows];
  };
};

// Four activations at element offset `off` of the activation buffer (kOob:
// zeros), kept as loaded (bf16 pairs stay packed, half the registers) until
// the conversion widens them.
template <bool BF16>
struct XRaw {
  using type = float4;
};
template <>
struct XRaw<true> {
  using type = uint2;
};

template <bool BF16>
__device__ __forceinline__ typename XRaw<BF16>::type load_x4(rsrc_t r, uint32_t off) {
  if constexpr (BF16) {
    return buf_load8(r, off == kOob ? kOob : 2u * off);
  } else {
    const uint4 raw = buf_load16(r, off == kOob ? kOob : 4u * off);
    return make_float4(__uint_as_float(raw.x), __uint_as_float(raw.y), __uint_as_float(raw.z),
                       __uint_as_float(raw.w));
  }
}

__device__ __forceinline__ float4 widen(const float4& v) { return v; }

__device__ __forceinline__ float4 widen(const uint2& raw) {
  return make_float4(bf16_bits_to_float(raw.x & 0xFFFFu), bf16_bits_to_float(raw.x >> 16),
                     bf16_bits_to_float(raw.y & 0xFFFFu), bf16_bits_to_float(raw.y >> 16));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, true));
}

// Exponent that maps a maximum |x| into [2^14, 2^15) (0 when all values are
// zero).
__device__ __forceinline__ int block_shift(float amax) {
  const int eb = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
  return amax > 0.0f ? 141 - eb : 0;
}

// Converts loaded activations of one chunk into operand layout.  Lane l owns
// values 4l .. 4l+3 of each 256-block: operand step s = (l % 16) / 2, lane
// group g = l / 16, halves 4*(l%2) .. +3.  One scale per token for the whole
// chunk (blocks past `nb` were loaded as zeros and do not move the maximum).
// Tokens at or past the live count `mt` and blocks past `nb` are skipped
// (uniform branches): their operand rows hold stale values, which only reach
// result rows that are never read.
__device__ __forceinline__ uint32_t pkrtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

__device__ __forceinline__ float lo_half(uint32_t v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v & 0xFFFFu)));
}

__device__ __forceinline__ float hi_half(uint32_t v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v >> 16)));
}

// Per-token maxima of non-negative values over the wavefront (MT = 4 or 8).
// Lane swaps between half-waves and between rows (permlane32/16) take the
// maximum of token pairs and halve the number of values per step; DPP max
// steps finish within rows.  Each token's maximum ends in one lane, which
// max_lanes finds once per kernel.
__device__ __forceinline__ float swap_max32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_max16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int MT>
__device__ __forceinline__ float token_max(const float (&am)[MT], int lane) {
  static_assert(MT == 4 || MT == 8, "token count");
  float w[MT / 2];
#pragma unroll
  for (int j = 0; j < MT / 2; ++j) w[j] = swap_max32(am[2 * j], am[2 * j + 1]);
  float x[MT / 4];
#pragma unroll
  for (int i = 0; i < MT / 4; ++i) x[i] = swap_max16(w[2 * i], w[2 * i + 1]);
  float y;
  if constexpr (MT == 4) {
    y = fmaxf(x[0], dpp<0x128>(x[0]));  // row_ror:8 (lane xor 8 within a row)
  } else {
    const bool b3 = (lane >> 3) & 1;    // lanes 8..15 of a row keep x1, 0..7 x0
    y = fmaxf(b3 ? x[1] : x[0], dpp<0x128>(b3 ? x[0] : x[1]));
  }
  y = fmaxf(y, dpp<0xB1>(y));   // quad_perm(1,0,3,2)
  y = fmaxf(y, dpp<0x4E>(y));   // quad_perm(2,3,0,1)
  y = fmaxf(y, dpp<0x114>(y));  // row_shr:4: lanes 4..7 of each half-row hold the result
  return y;
}

// Lane holding token t's maximum after token_max (uniform), found by running
// the same swaps on token indices.
template <int MT>
__device__ __forceinline__ void max_lanes(int lane, int (&tl)[MT]) {
  uint32_t w[MT / 2];
#pragma unroll
  for (int j = 0; j < MT / 2; ++j) w[j] = __builtin_amdgcn_permlane32_swap(2u * j, 2u * j + 1u, false, false)[0];
  uint32_t x[MT / 4];
#pragma unroll
  for (int i = 0; i < MT / 4; ++i) x[i] = __builtin_amdgcn_permlane16_swap(w[2 * i], w[2 * i + 1], false, false)[0];
  int tok;
  bool holder;
  if constexpr (MT == 4) {
    tok = static_cast<int>(x[0]);
    holder = (lane & 15) == 15;
  } else {
    tok = static_cast<int>((lane >> 3) & 1 ? x[1] : x[0]);
    holder = (lane & 7) == 7;
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const unsigned long long m = __ballot(holder && tok == t);
    tl[t] = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(m)));
  }
}

template <int MT, typename XT>
__device__ __forceinline__ void convert_chunk(WaveLds<MT>& L, const XT (&xv)[MT][WaveLds<MT>::kCH],
                                              int mt, int nb, int lane, const int (&tl)[MT]) {
  constexpr int CH = WaveLds<MT>::kCH;
  constexpr int R2 = WaveLds<MT>::kR2;
  constexpr int HR = R2 / 2;
  const int s = (lane & 15) >> 1;
  const int g = lane >> 4;
  const int half = lane & 1;
  // every token's maximum at once (tokens past `mt` were loaded as zeros)
  float am[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    float v = 0.f;
#pragma unroll
    for (int bi = 0; bi < CH; ++bi) {
      const float4 x = widen(xv[t][bi]);
      v = fmaxf(v, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
    am[t] = v;
  }
  const float tmax = token_max<MT>(am, lane);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t >= mt) break;
    const float amax = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tmax), tl[t]));
    const int sh = block_shift(amax);
#pragma unroll
    for (int bi = 0; bi < CH; ++bi) {
      if (bi >= nb) break;
      const float4 x = widen(xv[t][bi]);
      const float v0 = ldexpf(x.x, sh), v1 = ldexpf(x.y, sh);
      const float v2 = ldexpf(x.z, sh), v3 = ldexpf(x.w, sh);
      const uint32_t h01 = pkrtz(v0, v1), h23 = pkrtz(v2, v3);
      const uint32_t l01 = pkrtz(v0 - lo_half(h01), v1 - hi_half(h01));
      const uint32_t l23 = pkrtz(v2 - lo_half(h23), v3 - hi_half(h23));
      const int e = WaveLds<MT>::idx(bi, s, g, t);
      reinterpret_cast<uint2*>(&L.op[e])[half] = make_uint2(h01, h23);
      reinterpret_cast<uint2*>(&L.op[e + HR])[half] = make_uint2(l01, l23);
    }
    if (lane == 0) L.shift[t] = sh;
  }
}

// Eight quants (low nibbles of the two dwords) times sc as binary16: a byte
// permute builds 1024 + q and one fused (1024 + q) * sc - 1024 * sc per pair
// yields q * sc exactly.
__device__ __forceinline__ v8h weights8(uint32_t w0, uint32_t w1, v2h s, v2h o) {
  const uint32_t k64 = 0x64646464u;
  const uint32_t m0 = w0 & 0x0F0F0F0Fu, m1 = w1 & 0x0F0F0F0Fu;
  const v2h p0 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(k64, m0, 0x04010400u));
  const v2h p1 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(k64, m0, 0x04030402u));
  const v2h p2 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(k64, m1, 0x04010400u));
  const v2h p3 = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(k64, m1, 0x04030402u));
  const v2h r0 = __builtin_elementwise_fma(p0, s, o);
  const v2h r1 = __builtin_elementwise_fma(p1, s, o);
  const v2h r2 = __builtin_elementwise_fma(p2, s, o);
  const v2h r3 = __builtin_elementwise_fma(p3, s, o);
  return v8h{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

struct BlockRegs {
  uint4 h;   // header
  uint4 q0;  // quant bytes 32g .. 32g+15
  uint4 q1;  // quant bytes 32g+16 .. 32g+31
};

// The block at byte offset `off` of the resource, lane group g (kOob: zeros).
__device__ __forceinline__ void load_block(rsrc_t r, uint32_t off, int g, BlockRegs& b) {
  b.h = buf_load16(r, off);
  const uint32_t q = off + 32u * static_cast<uint32_t>(g);
  b.q0 = buf_load16(r, q + 16u);
  b.q1 = buf_load16(r, q + 32u);
}

// One block of one matrix: the main chain (cm) and the min term (cn).
template <int MT>
__device__ __forceinline__ void block_mfma(const BlockRegs& r, int g, const WaveLds<MT>& L, int bi,
                                           int arow, float& d, float& dmin, v4f& cm, v4f& cn) {
  d = half_bits_to_float(r.h.x & 0xFFFFu);
  dmin = half_bits_to_float(r.h.x >> 16);
  uint32_t sc0, mn0, sc1, mn1;
  scale_min_rt(r.h, 2 * g, sc0, mn0);
  scale_min_rt(r.h, 2 * g + 1, sc1, mn1);
  const _Float16 fs0 = static_cast<_Float16>(static_cast<float>(sc0));
  const _Float16 fs1 = static_cast<_Float16>(static_cast<float>(sc1));
  const _Float16 fo0 = static_cast<_Float16>(-1024.0f * static_cast<float>(sc0));
  const _Float16 fo1 = static_cast<_Float16>(-1024.0f * static_cast<float>(sc1));
  const v2h s0 = v2h{fs0, fs0}, o0 = v2h{fo0, fo0};
  const v2h s1 = v2h{fs1, fs1}, o1 = v2h{fo1, fo1};
  const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
  // min term: the K values of lane group g in steps 0..3 belong to sub-block
  // 2g, in steps 4..7 to sub-block 2g+1
  const _Float16 fm0 = static_cast<_Float16>(static_cast<float>(mn0));
  const _Float16 fm1 = static_cast<_Float16>(static_cast<float>(mn1));
  const v8h bm0 = v8h{fm0, fm0, fm0, fm0, fm0, fm0, fm0, fm0};
  const v8h bm1 = v8h{fm1, fm1, fm1, fm1, fm1, fm1, fm1, fm1};
  cm = v4f{0.f, 0.f, 0.f, 0.f};
  cn = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const v8h b = s < 4 ? weights8(w[2 * s], w[2 * s + 1], s0, o0)
                        : weights8(w[2 * (s - 4)] >> 4, w[2 * (s - 4) + 1] >> 4, s1, o1);
    const v8h av = __builtin_bit_cast(v8h, L.op[WaveLds<MT>::idx(bi, s, g, arow)]);
    cm = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b, cm, 0, 0, 0);
    cn = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, s < 4 ? bm0 : bm1, cn, 0, 0, 0);
  }
}

__device__ __forceinline__ void lds_fence() {
  // this wavefront's LDS writes complete before its later LDS reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int MT, bool GU, bool BF16, int W, int RT, bool SPLIT>
__global__ __launch_bounds__(64 * W) void gemv_mfma_kernel(GemvArgs a) {
  constexpr int CH = WaveLds<MT>::kCH;
  constexpr int R2 = WaveLds<MT>::kR2;
  constexpr int HR = R2 / 2;
  __shared__ Lds<MT, GU, W> lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // uniform in the wavefront; readfirstlane tells the compiler so, which keeps
  // the chunk loop's branches scalar (a vector branch around a load makes the
  // compiler wait for it at the join)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.k / kQK;
  // the output of a later split launch (the down pass of the FFN) starts at
  // zero: every workgroup clears a share of it
  if (a.zero_out != nullptr) {
    const int per = (a.zero_n + gridDim.x - 1) / gridDim.x;
    const int z1 = min(a.zero_n, (static_cast<int>(blockIdx.x) + 1) * per);
    for (int i = static_cast<int>(blockIdx.x) * per + tid; i < z1; i += 64 * W) a.zero_out[i] = 0.f;
  }

  const int mt = min(a.m, MT);  // live tokens (rows of x and y)
  int tl[MT];                   // lane of each token's maximum in token_max
  max_lanes<MT>(lane, tl);

  // this workgroup's RT tiles of 16 rows
  const int n0 = blockIdx.x * (RT * kRows);
  const int rows = min(RT * kRows, a.n - n0);
  const int nl = lane & 15;   // B operand weight row / A operand row / C column
  const int g = lane >> 4;    // lane group: K slots 8g .. 8g+7
  const int arow = nl & (R2 - 1);
  // the workgroup's rows of each matrix (at most 48 rows * 128 blocks * 144 bytes)
  const size_t wofs = static_cast<size_t>(n0) * K * kBlockBytes;
  const uint32_t wbytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(K) * kBlockBytes;
  const rsrc_t rg = make_rsrc(a.w + wofs, wbytes);
  const rsrc_t ru = GU ? make_rsrc(a.w_up + wofs, wbytes) : rg;
  // activations: offsets are element indices of valid tokens only, so the
  // resource is left unbounded
  const rsrc_t rx = make_rsrc(a.x, 0x7FFFFFFFu);

  // this workgroup's blocks (all of k, or split blockIdx.y), then this
  // wavefront's share of them
  const int ks0 = SPLIT ? static_cast<int>(blockIdx.y) * K / a.splits : 0;
  const int ksn = (SPLIT ? (static_cast<int>(blockIdx.y) + 1) * K / a.splits : K) - ks0;
  const int kb0 = ks0 + (wave * ksn) / W;
  const int kb1 = ks0 + ((wave + 1) * ksn) / W;

  // byte offset of block cb + bi of this lane's row in tile r (kOob past the
  // workgroup's rows or the chunk's nbb blocks)
  auto w_off = [&](int r, int cb, int bi, int nbb) -> uint32_t {
    const int row = r * kRows + nl;
    return row < rows && bi < nbb ? static_cast<uint32_t>(row * K + cb + bi) * kBlockBytes : kOob;
  };
  using XT = typename XRaw<BF16>::type;
  auto load_x = [&](int cb, int nbb, XT (&xv)[MT][CH]) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int bi = 0; bi < CH; ++bi) {
        const uint32_t off = t < mt && bi < nbb
                                 ? static_cast<uint32_t>(t * a.ldx + (cb + bi) * kQK + 4 * lane)
                                 : kOob;
        xv[t][bi] = load_x4<BF16>(rx, off);
      }
  };

  float yg[RT][4], yu[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) yg[r][i] = yu[r][i] = 0.f;
  WaveLds<MT>& L = lds.wave[wave];

  // Pipeline: the activations of chunk c+1 are loaded while chunk c is
  // multiplied, and the weight registers of a block are refilled as soon as
  // the block is consumed (with the same block of the next tile, or of tile
  // 0 of the next chunk after the last tile), so loads stay in flight across
  // tiles and chunks.
  int cb = kb0;
  int nb = min(CH, kb1 - cb);
  XT xv[MT][CH];
  load_x(cb, nb, xv);
  BlockRegs rgb[CH], rub[GU ? CH : 1];
#pragma unroll
  for (int bi = 0; bi < CH; ++bi) {
    const uint32_t off = w_off(0, cb, bi, nb);
    load_block(rg, off, g, rgb[bi]);
    if constexpr (GU) load_block(ru, off, g, rub[bi]);
  }
  // One chunk; HN: a next chunk exists (its activations and the weights of
  // its first tile are loaded here).  The last chunk is peeled off so that no
  // load sits under a branch whose result is used after it.
  auto chunk = [&](auto hn) {
    constexpr bool HN = decltype(hn)::value;
    // 1. activations -> operand layout in this wavefront's LDS
    convert_chunk<MT, XT>(L, xv, mt, nb, lane, tl);
    lds_fence();
    const int cn = cb + CH;
    const int nbn = HN ? min(CH, kb1 - cn) : 0;
    if constexpr (HN) load_x(cn, nbn, xv);
    int shs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) shs[i] = L.shift[(4 * g + i) & (HR - 1)];
    // 2. one MFMA chain per block, tile and matrix; C element i of this lane
    //    is row 4g + i: token (4g + i) % HR, hi half when 4g + i < HR, lo when
    //    below R2
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int bi = 0; bi < CH; ++bi) {
        if (bi < nb) {  // uniform
          float d, dmin;
          v4f cmv, cnv;
          block_mfma<MT>(rgb[bi], g, L, bi, arow, d, dmin, cmv, cnv);
#pragma unroll
          for (int i = 0; i < 4; ++i) yg[r][i] += ldexpf(fmaf(d, cmv[i], -dmin * cnv[i]), -shs[i]);
          if constexpr (GU) {
            block_mfma<MT>(rub[bi], g, L, bi, arow, d, dmin, cmv, cnv);
#pragma unroll
            for (int i = 0; i < 4; ++i) yu[r][i] += ldexpf(fmaf(d, cmv[i], -dmin * cnv[i]), -shs[i]);
          }
        }
        // refill the block's registers: next tile, or tile 0 of the next chunk
        if (r + 1 < RT || HN) {  // compile-time
          const uint32_t off = r + 1 < RT ? w_off(r + 1, cb, bi, nb) : w_off(0, cn, bi, nbn);
          load_block(rg, off, g, rgb[bi]);
          if constexpr (GU) load_block(ru, off, g, rub[bi]);
        }
      }
    }
    lds_fence();
    cb = cn;
    nb = nbn;
  };
  while (cb + CH < kb1) chunk(std::integral_constant<bool, true>{});  // uniform
  if (cb < kb1) chunk(std::integral_constant<bool, false>{});         // uniform

  // 3. add the W partial tiles of each row tile in a fixed order
  // C layout: lane holds rows 4g .. 4g+3 of weight row nl
  const int t = tid / kRows;
  const int rr = tid % kRows;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lds.red[0][wave][4 * g + i][nl] = yg[r][i];
      if constexpr (GU) lds.red[GU ? 1 : 0][wave][4 * g + i][nl] = yu[r][i];
    }
    __syncthreads();
    if (t < mt && r * kRows + rr < rows) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) s += lds.red[0][w][t][rr] + lds.red[0][w][HR + t][rr];
      if constexpr (SPLIT) {
        __hip_atomic_fetch_add(a.y + static_cast<size_t>(t) * a.ldy + n0 + r * kRows + rr, s, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      } else {
        float out = s;
        if constexpr (GU) {
          float su = 0.f;
#pragma unroll
          for (int w = 0; w < W; ++w)
            su += lds.red[GU ? 1 : 0][w][t][rr] + lds.red[GU ? 1 : 0][w][HR + t][rr];
          out = silu_mul(s, su);
        }
        a.y[static_cast<size_t>(t) * a.ldy + n0 + r * kRows + rr] = out;
      }
    }
  }
}

template <int MT, int W, int RT>
hipError_t dispatch_w(const GemvArgs& a, const dim3& grid, hipStream_t stream) {
  const bool gu = a.w_up != nullptr;
  const bool bf = a.x_bf16 != 0;
  if (gu) {
    if (bf) gemv_mfma_kernel<MT, true, true, W, RT, false><<<grid, dim3(64 * W), 0, stream>>>(a);
    else gemv_mfma_kernel<MT, true, false, W, RT, false><<<grid, dim3(64 * W), 0, stream>>>(a);
  } else {
    if (bf) gemv_mfma_kernel<MT, false, true, W, RT, false><<<grid, dim3(64 * W), 0, stream>>>(a);
    else gemv_mfma_kernel<MT, false, false, W, RT, false><<<grid, dim3(64 * W), 0, stream>>>(a);
  }
  return hipGetLastError();
}

// Tiles per workgroup: every workgroup converts its share of the activations
// once per chunk and reuses them for RT tiles of 16 rows, RT chosen so that
// about 256 workgroups cover all tiles (at most 3).  k is split over the
// wavefronts of a workgroup: eight (two per SIMD, so that one converts or
// multiplies while the other waits on memory; 128 KiB of LDS, one workgroup
// per CU) while all workgroups fit on the 256 CUs at once, four otherwise.
template <int MT, int RT>
hipError_t dispatch_rt(const GemvArgs& a, int tiles, hipStream_t stream) {
  const dim3 grid((tiles + RT - 1) / RT);
  if (static_cast<long long>(grid.x) * grid.y <= 256) return dispatch_w<MT, kWavesMax, RT>(a, grid, stream);
  return dispatch_w<MT, 4, RT>(a, grid, stream);
}

template <int MT>
hipError_t dispatch_m(const GemvArgs& a, hipStream_t stream) {
  const int tiles = (a.n + kRows - 1) / kRows;
  const int rt = (tiles + 255) / 256;
  if (rt <= 1) return dispatch_rt<MT, 1>(a, tiles, stream);
  if (rt == 2) return dispatch_rt<MT, 2>(a, tiles, stream);
  return dispatch_rt<MT, 3>(a, tiles, stream);
}

// Split k: tiles per workgroup with two workgroups per row group, about 256
// workgroups in all.
int split_rt(int tiles) { return tiles <= 128 ? 1 : 2; }

template <int MT, int RT>
hipError_t dispatch_split_rt(const GemvArgs& a, int tiles, hipStream_t stream) {
  // at most 256 tiles: at most 256 workgroups, eight wavefronts each
  const dim3 grid((tiles + RT - 1) / RT, 2);
  gemv_mfma_kernel<MT, false, false, kWavesMax, RT, true><<<grid, dim3(64 * kWavesMax), 0, stream>>>(a);
  return hipGetLastError();
}

template <int MT>
hipError_t dispatch_split(const GemvArgs& a, hipStream_t stream) {
  const int tiles = (a.n + kRows - 1) / kRows;
  if (split_rt(tiles) == 1) return dispatch_split_rt<MT, 1>(a, tiles, stream);
  return dispatch_split_rt<MT, 2>(a, tiles, stream);
}

}  // namespace

// Two splits when the rows give at most 256 tiles of 16 (without them every
// workgroup converts the activations of all of k for only 16 rows) and k has
// at least 16 blocks (8 per half: one per wavefront).
int gemv_mfma_splits(int m, int n, int k) {
  if (m < 2 || m > 8) return 1;
  const int tiles = (n + kRows - 1) / kRows;
  return tiles <= 256 && k / kQK >= 16 ? 2 : 1;
}

// Tokens are rounded up to 4 or 8 (the operand holds hi and lo halves of up
// to eight tokens either way).
hipError_t launch_gemv_mfma(const GemvArgs& a, hipStream_t stream) {
  if (a.splits > 1) {
    // one dense f32 matrix, y zeroed by the caller
    if (a.splits != 2 || a.w_up != nullptr || a.x_bf16 || a.ids != nullptr || (a.n + kRows - 1) / kRows > 256)
      return hipErrorInvalidValue;
    if (a.m <= 4) return dispatch_split<4>(a, stream);
    return dispatch_split<8>(a, stream);
  }
  if (a.m <= 4) return dispatch_m<4>(a, stream);
  return dispatch_m<8>(a, stream);
}

}  // namespace q4k
