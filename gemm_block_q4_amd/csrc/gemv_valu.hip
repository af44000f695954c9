// Dequant-fused Q4_K GEMV on the vector ALUs for one token, gfx950.
//
// "realizar -- q4k_gemv_cached_uses.rs", q4k_gemv_cached_async: y = W x with
// W in block_q4_K [n][k/256] and f32 x of length k (k divisible by 256);
// "realizar -- ffn.rs", fused_ffn_swiglu_gpu: the gate and up projections of
// one input followed by silu(gate) * up, done here in one pass.
//
// Activation-stationary layout.  A row of the matrix is cut into 4*(k/256)
// slices of 64 weights (one quarter g of a 256-block: quant bytes 32g..32g+31,
// low nibbles = sub-block 2g, high nibbles = sub-block 2g+1).  Each lane owns
// one slice position for the whole kernel; the wavefront walks its rows and at
// every row each lane streams its slice (two 16-byte loads) and its block's
// 16-byte header (the four lanes of a block load the same line) and adds
//   d*sc_{2g} * sum q x  +  d*sc_{2g+1} * sum q x  -  dmin*(m_{2g} X_{2g} + m_{2g+1} X_{2g+1})
// where X are the f32 sums of the slice's two halves of x.  Consecutive lanes
// own consecutive quarters, so a wavefront's loads cover 16 consecutive blocks
// of a row.
//
// Integer inner products.  The activations are fixed for the whole kernel, so
// the workgroup converts them once: each 64-value slice gets a power-of-two
// scale 2^e with every |x| < 2^e, and each value becomes the integer
// a = rint(x * 2^(21-e)), |a| <= 2^21 (21 significant bits relative to the
// slice maximum).  One FMA with the constant 1.5 * 2^23 leaves a + 2^22 in the
// low 23 bits of the f32 result; its three bytes u0, u1, u2 give
// a = u0 + 2^8 u1 + 2^16 (u2 - 64), stored as two unsigned byte planes and one
// signed plane (u2 - 64 lies in [-32, 32]).  A masked nibble word is four
// bytes below 16, so four weights times one plane are one v_dot4 (unsigned
// for planes 0, 1, signed for plane 2), and the three plane sums of a
// sub-block combine exactly in int32 as S0 + 2^8 S1 + 2^16 S2, scaled by
// 2^(e-21).  No weight is ever converted to floating point.
//
// Latency: each thread loads its share of the activations first and the
// weight loads of the next PF rows right behind them (loads return in order);
// the workgroup writes the digits to LDS (one barrier), every lane copies its
// slice's 48 digit words to registers, and the row loop then consumes weights
// as they stream in.  A row that fits one wavefront is reduced with DPP lane
// permutes and stored directly; wider rows add their per-wavefront sums in LDS
// at the end.  The summation order is fixed (deterministic).
//
// MoE ("micro_moe.rs", DirectNvFp4MoeBf16::execute): the same kernel runs one
// (token, slot) pair per grid row on that pair's expert (gate/up), and
// moe_down_kernel below runs a token's slots on one wavefront each and adds
// them with the routing weights (down projection plus the combine).
#include <algorithm>

#include "lane_reduce.hpp"
#include "q4k_device.hpp"
#include "q4k_internal.hpp"
#include "slice_dot.hpp"

namespace q4k {

namespace {

constexpr int kThreadsMax = 768;  // the wide layout: 12 wavefronts
constexpr int kThreadsNarrow = 512;
constexpr int kWavesNarrow = 4;  // wavefronts per workgroup when a row fits one wavefront
constexpr int kWavesWide = 12;   // at most this many when a row spans wavefronts
constexpr size_t kLdsMax = 160 * 1024;

// Launch geometry (all per workgroup):
//   lanes per row  lpr = 4 * (k/256) slices, rounded up to a power of two when
//   a row fits one wavefront (so rows are aligned lane segments);
//   wr   = wavefronts per row (1 when lpr <= 64);
//   rpw  = rows per wavefront per step (64 / lpr when wr == 1, else 1);
//   step = rows per workgroup per step; rows = rows per workgroup.
// The kernel divides by none of them: lpr_log = log2(lpr) when wr == 1, and
// for wr > 1 nibble w of wslot / wpart holds w / wr and w % wr (up to 12
// wavefronts).
struct Geo {
  int lpr, wr, rpw, waves, step, rows;
  int lpr_log;
  uint64_t wslot, wpart;
};

// Row layouts: rows narrower than a wavefront (segments of lpr lanes), rows of
// exactly one wavefront, rows spanning wavefronts.
enum Layout { kNarrow = 0, kOneWave = 1, kWide = 2 };

// Kernel modes: one dense matrix (grid.y = 1), or the MoE pass (grid.y =
// (token, slot) pair p: the rows of expert ids[p] on x row p / top_k (gate /
// up) or p (down), output row p; a pair with an id outside [0, n_experts)
// does nothing).  Every pair is independent, so an expert chosen by several
// tokens streams its rows once per pair (from L2 when the pairs' workgroups
// run close together), and no workgroup runs passes back to back.
enum Mode { kDense = 0, kPair = 1 };

template <bool GU, bool BF16, int MODE, int LAYOUT, int XU, int PF>
__global__ __launch_bounds__(LAYOUT == kWide ? kThreadsMax : kThreadsNarrow) void gemv_d4_kernel(GemvArgs a, Geo geo) {
  constexpr bool WIDE = LAYOUT == kWide;
  constexpr bool SEG64 = LAYOUT != kNarrow;
  // rows of one or more whole wavefronts reduce their PF (non-GU) or 2 * PF
  // (GU: gate and up) values per lane together: 4 or 8 of them
  constexpr int NV = GU ? 2 * PF : PF;
  static_assert(!SEG64 || NV == 2 || NV == 4 || NV == 8, "one-wave reduction takes two, four or eight values");
  extern __shared__ __attribute__((aligned(16))) uint32_t smem_u[];
  const int K = a.k >> 8;  // blocks per row
  const int S = 4 * K;     // slices per row
  const int units = 4 * S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nthr = geo.waves * 64;
  // every argument the weight stream needs, fetched in one batch of scalar
  // loads (otherwise the compiler spreads them over dependent round trips
  // ahead of the first weight load)
  asm volatile("" ::"s"(a.w), "s"(a.w_up), "s"(a.x), "s"(a.k), "s"(a.n), "s"(geo.rows), "s"(geo.step),
               "s"(geo.lpr_log), "s"(geo.wslot), "s"(geo.wpart));

  // this lane's row slot (within a step) and slice position; for rows of one
  // or more whole wavefronts the row slot is uniform in the wavefront
  int rslot, slice;
  if constexpr (LAYOUT == kNarrow) {
    rslot = wave * geo.rpw + (lane >> geo.lpr_log);
    slice = lane & ((1 << geo.lpr_log) - 1);
  } else if constexpr (LAYOUT == kOneWave) {
    rslot = wave;
    slice = lane;
  } else {
    rslot = static_cast<int>((geo.wslot >> (4 * wave)) & 15u);
    slice = static_cast<int>((geo.wpart >> (4 * wave)) & 15u) * 64 + lane;
  }
  const bool lane_ok = slice < S && rslot < geo.step;
  const int b = lane_ok ? slice >> 2 : 0;
  const int g = lane & 3;  // == slice & 3: S is a multiple of 4 and segments are aligned
  const FieldSel fsel = field_sel(g);
  const uint32_t qoff = 16u + 32u * static_cast<uint32_t>(g);

  // step it holds rows it*step .. it*step+step-1 of the workgroup; it exists
  // while it*step < rows
  const int row0 = blockIdx.x * geo.rows;
  const int rows = min(geo.rows, a.n - row0);
  const uint32_t wbytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(K) * kBlockBytes;
  // Products of uniform values pass through an opaque scalar move: the
  // compiler would otherwise fold them with a lane value into a 64-bit
  // multiply-add whose (unused) high addend register may be a load in
  // flight, and wait for it (it sees through readfirstlane of a scalar).
  auto uni = [](int v) -> int {
    int r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "s"(v));
    return r;
  };
  // Byte offset of this lane's block in step it: base + it * stride (adds
  // only).  Rows past the workgroup's last start at or past the resource's
  // size and read zeros; a lane past the row's last slice starts at kOob
  // (2^31).  Every offset stays below 2^32: the workgroup's bytes and the
  // PF steps past its end stay below 2^31 (make_geo), so nothing wraps and
  // no load needs a branch or a per-row select.
  const uint32_t stride = static_cast<uint32_t>(geo.step * K) * kBlockBytes;
  const uint32_t base = lane_ok ? static_cast<uint32_t>(rslot * K + b) * kBlockBytes : kOob;
  // Unit j of this thread's activation units (XU of them, XU * nthr >= units
  // by construction of the launch).
  auto unit_off = [&](int u, int c) -> uint32_t {
    return u < units ? static_cast<uint32_t>(16 * u + 4 * c) : kOob;
  };
  uint32_t* dig = smem_u;                                                    // 12 planes
  float* xinfo = reinterpret_cast<float*>(smem_u + xinfo_offset(S));          // [S][4]
  float* part = reinterpret_cast<float*>(smem_u + x_words(S));                   // [GU?2:1][rows][wr]
  const int seg_mask = SEG64 ? 63 : (1 << geo.lpr_log) - 1;

  // rows of whole wavefronts: which of the NV reduced values each lane ends
  // up holding (row_reduce<NV>), and the lanes that hold values 0 .. NV-1
  int hold_tok = 0;
  bool holder = false;
  int hl[NV];
#pragma unroll
  for (int t = 0; t < NV; ++t) hl[t] = 63;
  if constexpr (SEG64) {
    token_map<NV>(lane, hold_tok, holder);
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const uint64_t m = __ballot(holder && hold_tok == t);
      hl[t] = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(m)));
    }
  }

  // One pass over the workgroup's rows of one matrix for one activation row;
  // writes y row `yrow`.
  auto pass = [&](size_t mofs, int xrow, int yrow) {
    const size_t wofs = mofs + static_cast<size_t>(row0) * K * kBlockBytes;
    const rsrc_t rg = make_rsrc(a.w + wofs, wbytes);
    const rsrc_t ru = GU ? make_rsrc(a.w_up + wofs, wbytes) : rg;
    const size_t xel = static_cast<size_t>(xrow) * a.ldx;
    const rsrc_t rx = BF16 ? make_rsrc(static_cast<const uint16_t*>(a.x) + xel, 2u * a.k)
                           : make_rsrc(static_cast<const float*>(a.x) + xel, 4u * a.k);
    float* yout = a.y + static_cast<size_t>(yrow) * a.ldy + row0;

    // 1. this thread's activation units, loaded before any weight
    float4 xr[XU][4];
#pragma unroll
    for (int j = 0; j < XU; ++j) {
      // a wavefront whose units all lie past the end issues no loads (a
      // uniform branch; zero-returning loads would still take texture-path
      // slots ahead of the weights)
      if (wave * 64 + j * nthr < units) {
#pragma unroll
        for (int c = 0; c < 4; ++c) xr[j][c] = load_x4<BF16>(rx, unit_off(tid + j * nthr, c));
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) xr[j][c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }

    // Every wavefront issues its activation loads before any weight load:
    // the compute unit's texture path (64 B/clk) serves loads roughly in
    // issue order, and the activations, needed first, would otherwise queue
    // behind other wavefronts' weight loads (0.3 us on 4096 x 4096).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // 2. weight loads of the first PF steps
    RawSlice sg[PF], su[GU ? PF : 1];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const uint32_t off = base + static_cast<uint32_t>(uni(p * static_cast<int>(stride)));
      load_slice(rg, off, qoff, sg[p]);
      if constexpr (GU) load_slice(ru, off, qoff, su[p]);
    }

    // 3. activations -> digits in LDS, once per workgroup (the loop bounds are
    //    uniform, so every quad converts together)
#pragma unroll
    for (int j = 0; j < XU; ++j) {
      const int u = tid + j * nthr;
      convert_unit(xr[j], u, u < units, S, dig, xinfo);
    }
    // A barrier without a memory fence: the digits are LDS writes, complete
    // at lgkmcnt(0), and a fence would also wait for the weight loads in
    // flight.
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    XSlice xs;
    {
      read_digits(dig, S, lane_ok ? slice : 0, xs.dg);
      const float4 inf = *reinterpret_cast<const float4*>(xinfo + 4 * (lane_ok ? slice : 0));
      xs.scale = inf.x; xs.sum0 = inf.y; xs.sum1 = inf.z;
    }

    // 4. row loop: consume step p while steps p+1 .. p+PF-1 are in flight.
    //    The loads are never under a branch (rows past the end read zeros),
    //    the last group issues none, and lanes past the row's end give 0.
    auto finish = [&](float (&o)[PF], float (&ou)[PF], int it0) {
      if constexpr (!SEG64) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
          o[p] = segment_sum_rt(o[p], seg_mask + 1);
          if constexpr (GU) ou[p] = segment_sum_rt(ou[p], seg_mask + 1);
        }
#pragma unroll
        for (int p = 0; p < PF; ++p) {
          const int r = uni((it0 + p) * geo.step) + rslot;
          // the segment's last lane holds the row sum (it may be a padding lane)
          if (rslot < geo.step && r < rows && (lane & seg_mask) == seg_mask) {
            float out = o[p];
            if constexpr (GU) out = silu_mul(o[p], ou[p]);
            yout[r] = out;
          }
        }
      } else {
        // NV values per lane -> NV totals (row_reduce<NV>): non-GU the PF
        // steps' rows, GU the PF steps' gate rows, then their up rows
        float v[NV];
#pragma unroll
        for (int p = 0; p < PF; ++p) {
          v[p] = o[p];
          if constexpr (GU) v[PF + p] = ou[p];
        }
        const float tot = row_reduce<NV>(v, lane);
        if constexpr (!GU) {
          const int r = uni(it0 * geo.step) + hold_tok * geo.step + rslot;
          if (holder && r < rows) {
            if constexpr (!WIDE) yout[r] = tot;
            else part[r * geo.wr + (slice >> 6)] = tot;
          }
        } else if constexpr (!WIDE) {
          // lane p (< PF) gathers the gate and up totals of step it0 + p
          // from their holders (uniform lane indices) and stores silu * up
          float gt = 0.f, ut = 0.f;
#pragma unroll
          for (int p = 0; p < PF; ++p) {
            const float g_p = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tot), hl[p]));
            const float u_p = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tot), hl[PF + p]));
            gt = lane == p ? g_p : gt;
            ut = lane == p ? u_p : ut;
          }
          const int r = uni(it0 * geo.step) + lane * geo.step + rslot;
          if (lane < PF && r < rows) yout[r] = silu_mul(gt, ut);
        } else {
          const int p = hold_tok % PF;
          const int r = uni(it0 * geo.step) + p * geo.step + rslot;
          if (holder && r < rows) part[((hold_tok / PF) * rows + r) * geo.wr + (slice >> 6)] = tot;
        }
      }
    };
    int it0 = 0;
    uint32_t next = base + PF * stride;  // offset of step it0 + PF
    for (; (it0 + PF) * geo.step < rows; it0 += PF, next += PF * stride) {  // uniform; a later group exists
      float o[PF], ou[PF];
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        o[p] = slice_dot(sg[p], fsel, xs);
        ou[p] = 0.f;
        if constexpr (GU) ou[p] = slice_dot(su[p], fsel, xs);
        const uint32_t off = next + static_cast<uint32_t>(uni(p * static_cast<int>(stride)));
        load_slice(rg, off, qoff, sg[p]);
        if constexpr (GU) load_slice(ru, off, qoff, su[p]);
      }
      finish(o, ou, it0);
    }
    {  // the last group: nothing left to load
      float o[PF], ou[PF];
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        o[p] = 0.f;
        ou[p] = 0.f;
        if ((it0 + p) * geo.step < rows) {  // uniform
          o[p] = slice_dot(sg[p], fsel, xs);
          if constexpr (GU) ou[p] = slice_dot(su[p], fsel, xs);
        }
      }
      finish(o, ou, it0);
    }
    if constexpr (WIDE) {
      __syncthreads();
      // 5. rows that span wavefronts: add the per-wavefront sums in order
      for (int r = tid; r < rows; r += nthr) {
        float s = 0.f, su_ = 0.f;
        for (int w = 0; w < geo.wr; ++w) {
          s += part[r * geo.wr + w];
          if constexpr (GU) su_ += part[(rows + r) * geo.wr + w];
        }
        float out = s;
        if constexpr (GU) out = silu_mul(s, su_);
        yout[r] = out;
      }
    }
  };

  if constexpr (MODE == kDense) {
    pass(0, 0, 0);
  } else {
    const int pr = blockIdx.y;
    const int e = a.ids[pr];
    if (e < 0 || e >= a.n_experts) return;  // uniform, before any barrier
    pass(static_cast<size_t>(e) * a.mat_bytes, a.x_by_token ? pr / a.top_k : pr, pr);
  }
}

// MoE down projection with the combine folded in.  Workgroup (row group, token
// t) of W wavefronts; wavefront w takes slots w, w + W, ... of t.  For slot s
// (pair p = t * top_k + s, expert ids[p]) the wavefront converts h row p into
// its own LDS digits and runs the workgroup's rows of that expert (a row fits
// one wavefront: k <= 4096); row results land in res[s][row].  Finally each
// row adds wts[p] * res[s][row] over the valid slots in slot order
// (deterministic) and writes y[t][row].  No pair buffer and no combine pass.
template <int LAYOUT, int XU>
__global__ __launch_bounds__(kThreadsNarrow) void moe_down_kernel(GemvArgs a, Geo geo) {
  constexpr bool SEG64 = LAYOUT != kNarrow;
  constexpr int PF = 4;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem_u[];
  const int K = a.k >> 8;
  const int S = 4 * K;
  const int units = 4 * S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nthr = geo.waves * 64;
  const int t = blockIdx.y;
  const int row0 = blockIdx.x * geo.rows;
  const int rows = min(geo.rows, a.n - row0);
  const uint32_t wbytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(K) * kBlockBytes;

  // per-wavefront digits, then res[top_k][geo.rows]
  uint32_t* dig = smem_u + static_cast<size_t>(wave) * x_words(S);
  float* xinfo = reinterpret_cast<float*>(dig + xinfo_offset(S));
  float* res = reinterpret_cast<float*>(smem_u + static_cast<size_t>(geo.waves) * x_words(S));

  const int rslot = lane >> geo.lpr_log;  // row within a step (geo.rpw rows per step)
  const int slice = lane & ((1 << geo.lpr_log) - 1);
  const bool lane_ok = slice < S;
  const int b = lane_ok ? slice >> 2 : 0;
  const int g = lane & 3;
  const FieldSel fsel = field_sel(g);
  const uint32_t qoff = 16u + 32u * static_cast<uint32_t>(g);
  const int seg_mask = SEG64 ? 63 : (1 << geo.lpr_log) - 1;
  const int step = geo.rpw;  // rows per wavefront step
  auto uni = [](int v) -> int {
    int r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "s"(v));
    return r;
  };
  // as in gemv_d4_kernel: rows past the end read zeros through the resource
  // size, lanes past the row's end start at kOob
  const uint32_t stride = static_cast<uint32_t>(step * K) * kBlockBytes;
  const uint32_t base = lane_ok ? static_cast<uint32_t>(rslot * K + b) * kBlockBytes : kOob;

  for (int sl = wave; sl < a.top_k; sl += geo.waves) {  // uniform in the wavefront
    const int pr = t * a.top_k + sl;
    const int e = a.ids[pr];
    if (e < 0 || e >= a.n_experts) continue;  // skipped again in the sum
    const size_t wofs = static_cast<size_t>(e) * a.mat_bytes + static_cast<size_t>(row0) * K * kBlockBytes;
    const rsrc_t rg = make_rsrc(a.w + wofs, wbytes);
    const rsrc_t rx = make_rsrc(static_cast<const float*>(a.x) + static_cast<size_t>(pr) * a.ldx, 4u * a.k);
    // 1. this lane's activation units (XU * 64 >= units), then the weights
    float4 xr[XU][4];
#pragma unroll
    for (int j = 0; j < XU; ++j) {
      const int u = lane + 64 * j;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        xr[j][c] = load_x4<false>(rx, u < units ? static_cast<uint32_t>(16 * u + 4 * c) : kOob);
    }
    RawSlice sg[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p)
      load_slice(rg, base + static_cast<uint32_t>(uni(p * static_cast<int>(stride))), qoff, sg[p]);
    // 2. digits of h row pr in this wavefront's LDS (the wavefront's own
    //    writes: complete at lgkmcnt(0))
#pragma unroll
    for (int j = 0; j < XU; ++j) {
      const int u = lane + 64 * j;
      convert_unit(xr[j], u, u < units, S, dig, xinfo);
    }
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    XSlice xs;
    {
      read_digits(dig, S, lane_ok ? slice : 0, xs.dg);
      const float4 inf = *reinterpret_cast<const float4*>(xinfo + 4 * (lane_ok ? slice : 0));
      xs.scale = inf.x; xs.sum0 = inf.y; xs.sum1 = inf.z;
    }
    // 3. the workgroup's rows of expert e, PF steps in flight
    float* rs = res + static_cast<size_t>(sl) * geo.rows;
    auto finish = [&](float (&o)[PF], int it0) {
#pragma unroll
      for (int p = 0; p < PF; ++p) o[p] = SEG64 ? segment_sum<64>(o[p]) : segment_sum_rt(o[p], seg_mask + 1);
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        const int r = uni((it0 + p) * step) + rslot;
        if (r < rows && (lane & seg_mask) == seg_mask) rs[r] = o[p];
      }
    };
    int it0 = 0;
    uint32_t next = base + PF * stride;
    for (; (it0 + PF) * step < rows; it0 += PF, next += PF * stride) {
      float o[PF];
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        o[p] = slice_dot(sg[p], fsel, xs);
        load_slice(rg, next + static_cast<uint32_t>(uni(p * static_cast<int>(stride))), qoff, sg[p]);
      }
      finish(o, it0);
    }
    {
      float o[PF];
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        o[p] = 0.f;
        if ((it0 + p) * step < rows) o[p] = slice_dot(sg[p], fsel, xs);
      }
      finish(o, it0);
    }
    // this wavefront's digits are rewritten by its next slot: its lanes are
    // done reading them (registers) once the loop above has run
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // 4. y[t][row] = sum over valid slots, in slot order
  for (int r = tid; r < rows; r += nthr) {
    float acc = 0.f;
    for (int sl = 0; sl < a.top_k; ++sl) {
      const int pr = t * a.top_k + sl;
      const int e = a.ids[pr];
      if (e >= 0 && e < a.n_experts) acc = fmaf(a.wts[pr], res[static_cast<size_t>(sl) * geo.rows + r], acc);
    }
    a.y[static_cast<size_t>(t) * a.ldy + row0 + r] = acc;
  }
}

// LDS bytes: digits and slice info, and the row partials when a row spans
// wavefronts.
size_t lds_bytes(const Geo& geo, int k, bool gu) {
  size_t words = x_words(4 * (k / kQK));
  if (geo.wr > 1) words += static_cast<size_t>(gu ? 2 : 1) * geo.rows * geo.wr;
  return words * sizeof(uint32_t);
}

Geo make_geo(int n, int k, int slots, bool gu, int mode) {
  Geo g{};
  const int K = k / kQK;
  const int l = 4 * K;
  if (l <= 64) {
    g.lpr = 1;
    g.lpr_log = 0;
    while (g.lpr < l) {
      g.lpr <<= 1;
      ++g.lpr_log;
    }
    g.wr = 1;
    g.rpw = 64 / g.lpr;
    g.waves = kWavesNarrow;
    g.step = g.waves * g.rpw;
  } else {
    g.lpr = l;
    g.wr = (l + 63) / 64;
    g.rpw = 1;
    g.waves = g.wr * (g.wr >= kWavesWide ? 1 : kWavesWide / g.wr);  // whole rows
    g.step = g.waves / g.wr;
    for (int w = 0; w < g.waves; ++w) {  // waves <= 12: one nibble each
      g.wslot |= static_cast<uint64_t>(w / g.wr) << (4 * w);
      g.wpart |= static_cast<uint64_t>(w % g.wr) << (4 * w);
    }
  }
  // rows per workgroup: about 256 workgroups over all slots, whole steps,
  // and no more row partials than fit next to the digits in LDS
  long long want = (static_cast<long long>(n) * slots + 255) / 256;
  if (want > n) want = n;
  if (want < g.step) want = g.step;
  g.rows = static_cast<int>((want + g.step - 1) / g.step * g.step);
  // MoE pairs: two prefetch groups per workgroup (the many pairs fill the
  // chip; a second group reuses the workgroup's activation conversion:
  // 24.1-24.5 us for the 64-expert top-8 FFN against 26.3-26.7 with one, and
  // 25.3-27.4 with three to eight); the kernel's steps in flight
  const int pf = g.wr > 1 ? (gu ? 1 : 2) : (gu ? 2 : 4);
  if (mode == kPair && g.rows > 2 * pf * g.step) g.rows = 2 * pf * g.step;
  // a workgroup's bytes stay below 2^30, so that its offsets, the PF steps
  // issued past its last row and the kOob start of lanes past the row's end
  // all stay below 2^32
  const int cap_bytes = static_cast<int>(((size_t{1} << 30) - 1) / (static_cast<size_t>(K) * kBlockBytes)) /
                        g.step * g.step;
  if (g.rows > cap_bytes) g.rows = cap_bytes;
  // (per row: the partials of a row that spans wavefronts)
  const size_t per_row = g.wr > 1 ? static_cast<size_t>(gu ? 2 : 1) * g.wr : 0;
  if (per_row > 0) {
    const size_t free_words = kLdsMax / sizeof(uint32_t) - x_words(l);
    const int cap = static_cast<int>(free_words / per_row) / g.step * g.step;
    if (g.rows > cap) g.rows = cap;
  }
  return g;
}

template <bool GU, bool BF16, int MODE, int LAYOUT, int XU>
hipError_t launch_layout(const GemvArgs& a, const Geo& geo, size_t lds, int grid_y, hipStream_t stream) {
  // steps in flight per wavefront: 4 rows (two of gate and of up), 2 (one
  // of each) when a row spans wavefronts: 12 wavefronts then keep about as
  // many bytes in flight per compute unit as 4 wavefronts of whole rows
  constexpr int PF = LAYOUT == kWide ? (GU ? 1 : 2) : (GU ? 2 : 4);
  auto kern = gemv_d4_kernel<GU, BF16, MODE, LAYOUT, XU, PF>;
  const hipError_t e = lds_opt_in(reinterpret_cast<const void*>(kern), lds);
  if (e != hipSuccess) return e;
  const dim3 grid((a.n + geo.rows - 1) / geo.rows, grid_y);
  kern<<<grid, dim3(geo.waves * 64), lds, stream>>>(a, geo);
  return hipGetLastError();
}

template <bool GU, bool BF16, int MODE>
hipError_t launch_mode(const GemvArgs& a, hipStream_t stream) {
  // grid rows: the MoE pairs, or the single dense matrix
  const int grid_y = MODE == kPair ? a.pairs : 1;
  const Geo geo = make_geo(a.n, a.k, grid_y, GU, MODE);
  const size_t lds = lds_bytes(geo, a.k, GU);
  if (geo.rows < geo.step || lds > kLdsMax) return hipErrorInvalidValue;
  // activation units (16 values) per thread: one when a row fits a wavefront
  // (at most 256 units for 256 threads), else one, two or four (k <= 32768
  // keeps units <= 4 * threads for every row width).  The fewest that cover
  // the units: a unit past the end still issues its (zero-returning) loads,
  // which queue ahead of the weight loads (k = 11008 on 12 wavefronts: 688
  // units, one per thread, 7.6 us against 8.1 with two).
  const int units = 16 * (a.k / kQK);
  const int nthr = geo.waves * 64;
  if (geo.wr > 1) {
    if (units <= nthr) return launch_layout<GU, BF16, MODE, kWide, 1>(a, geo, lds, grid_y, stream);
    if (units <= 2 * nthr) return launch_layout<GU, BF16, MODE, kWide, 2>(a, geo, lds, grid_y, stream);
    if (units <= 4 * nthr) return launch_layout<GU, BF16, MODE, kWide, 4>(a, geo, lds, grid_y, stream);
    return hipErrorInvalidValue;
  }
  if (units > nthr) return hipErrorInvalidValue;
  if (geo.lpr == 64) return launch_layout<GU, BF16, MODE, kOneWave, 1>(a, geo, lds, grid_y, stream);
  return launch_layout<GU, BF16, MODE, kNarrow, 1>(a, geo, lds, grid_y, stream);
}

template <bool GU, bool BF16>
hipError_t launch_d4(const GemvArgs& a, hipStream_t stream) {
  if (a.ids != nullptr) return launch_mode<GU, BF16, kPair>(a, stream);
  return launch_mode<GU, BF16, kDense>(a, stream);
}

}  // namespace

// One token (or the MoE passes, one routed pair at a time) and k up to 32768:
// at most 8 wavefronts per row, and the digits of all activations (208 bytes
// per 64 values, 104 KiB at k = 32768) fit in LDS.
bool gemv_valu_fits(int m, int k) { return m == 1 && k <= 32768; }

// MoE down projection with the combine (rows that fit one wavefront, and the
// per-wavefront digits and per-slot row results within LDS);
// hipErrorNotSupported otherwise.
hipError_t launch_moe_down(const GemvArgs& a, hipStream_t stream) {
  constexpr int PF = 4;
  const int K = a.k / kQK;
  const int l = 4 * K;
  if (l > 64 || a.w_up != nullptr || a.x_bf16 || a.top_k < 1) return hipErrorNotSupported;
  Geo g{};
  g.lpr = 1;
  while (g.lpr < l) {
    g.lpr <<= 1;
    ++g.lpr_log;
  }
  g.wr = 1;
  g.rpw = 64 / g.lpr;
  g.waves = std::min(a.top_k, 8);
  g.step = g.rpw;
  g.rows = g.rpw * PF * 2;  // two prefetch groups per slot: one conversion serves more rows
  const size_t lds = (static_cast<size_t>(g.waves) * x_words(l) +
                      static_cast<size_t>(a.top_k) * g.rows) * sizeof(uint32_t);
  if (lds > kLdsMax) return hipErrorNotSupported;
  const int xu = (16 * K + 63) / 64;  // activation units per lane (1..4)
  const dim3 grid((a.n + g.rows - 1) / g.rows, a.m);
  auto go = [&](auto kern) -> hipError_t {
    const hipError_t e = lds_opt_in(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
    kern<<<grid, dim3(g.waves * 64), lds, stream>>>(a, g);
    return hipGetLastError();
  };
  const bool one = g.lpr == 64;
  switch (xu) {
    case 1: return one ? go(moe_down_kernel<kOneWave, 1>) : go(moe_down_kernel<kNarrow, 1>);
    case 2: return one ? go(moe_down_kernel<kOneWave, 2>) : go(moe_down_kernel<kNarrow, 2>);
    case 3: return one ? go(moe_down_kernel<kOneWave, 3>) : go(moe_down_kernel<kNarrow, 3>);
    default: return one ? go(moe_down_kernel<kOneWave, 4>) : go(moe_down_kernel<kNarrow, 4>);
  }
}

hipError_t launch_gemv_valu(const GemvArgs& a, hipStream_t stream) {
  const bool gu = a.w_up != nullptr;
  const bool bf = a.x_bf16 != 0;
  if (gu) return bf ? launch_d4<true, true>(a, stream) : launch_d4<true, false>(a, stream);
  return bf ? launch_d4<false, true>(a, stream) : launch_d4<false, false>(a, stream);
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  if (a.ids != nullptr || gemv_valu_fits(a.m, a.k)) return launch_gemv_valu(a, stream);
  return launch_gemv_mfma(a, stream);
}

}  // namespace q4k
