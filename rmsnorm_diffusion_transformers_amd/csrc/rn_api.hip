// rn_api.hip -- the C ABI declared in include/resnorm.h: argument validation,
// launch planning and the enqueue of the gfx950 row kernels.
//
// Host-side rules (all checked before anything is enqueued):
//   * operand presence must match the flags (a present-but-unflagged operand
//     is an error, as is a flagged-but-missing one), so a caller cannot
//     silently get a different specialisation than it asked for;
//   * D % 8 == 0 (16-byte vectors), 8 <= D <= RN_D_MAX, every pointer 16-byte
//     aligned, B * L < 2^31 (32-bit row indices in the kernels);
//   * a per-frame layout needs 1 <= F and L % F == 0 (frame-major tokens:
//     49 frames x 3600 tokens in sglang PR #36349, "Microbenchmark");
//   * eps is honoured and must be finite and >= 0 (the prior-art kernel
//     ignored it and hard-coded 1e-6: sglang PR #33144, "Modifications");
//   * an empty problem (B * L == 0) returns OK without a launch (the prior art
//     had no empty-tensor guard: sglang PR #33144, "Known gaps").
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>

#include <cmath>

#include "../../include/resnorm.h"
#include "rn_args.h"

namespace {

thread_local char g_err[512];

rn_status fail(rn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

// Operands by id, for the overlap check and its messages.
enum Operand { kY, kResidualOut, kYScale, kX, kResidual, kGate, kWeight, kBias, kScale, kShift, kNumOperands };
const char* const kOperandName[kNumOperands] = {"y",    "residual_out", "y_scale", "x",     "residual",
                                                "gate", "weight",       "bias",    "scale", "shift"};

struct Extent {
  int id;
  uintptr_t lo;
  uintptr_t hi;  // one past the end
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t layout_rows(rn_layout lay, int64_t B, int64_t L) {
  switch (lay.kind) {
    case RN_BCAST: return 1;
    case RN_ROW: return B * L;
    case RN_FRAME: return B * (int64_t)lay.frames;
    default: return -1;
  }
}

rn_status check_layout(const char* what, rn_layout lay, int64_t L) {
  if (lay.kind != RN_BCAST && lay.kind != RN_ROW && lay.kind != RN_FRAME)
    return fail(RN_EINVAL, "%s layout kind %d is not RN_BCAST, RN_ROW or RN_FRAME", what, (int)lay.kind);
  if (lay.kind == RN_FRAME) {
    if (lay.frames < 1) return fail(RN_EINVAL, "%s layout RN_FRAME needs frames >= 1 (got %d)", what, (int)lay.frames);
    if (L % lay.frames != 0)
      return fail(RN_EINVAL, "%s layout RN_FRAME needs L %% frames == 0 (L=%lld, frames=%d)", what,
                  (long long)L, (int)lay.frames);
  }
  return RN_OK;
}

struct Problem {
  bool fused;
  int affine_dtype;  // RN_DTYPE_BF16 or RN_DTYPE_F32
  int y_dtype;       // RN_DTYPE_BF16, RN_DTYPE_F32 or RN_DTYPE_FP8_E4M3
  float* y_scale;
  void* y;
  void* residual_out;
  const void* x;
  const void* residual;
  const void* gate;
  const void* weight;
  const void* bias;
  const void* scale;
  const void* shift;
  int64_t B, L, D;
  uint32_t flags;
  rn_layout gate_layout, ss_layout;
  float eps;
};

rn_status check_shape(int64_t B, int64_t L, int64_t D, uint32_t flags, bool fused) {
  const uint32_t known = RN_RMS | RN_GATE | RN_WEIGHT | RN_BIAS;
  if (flags & ~known) return fail(RN_EINVAL, "unknown flag bits 0x%x", flags & ~known);
  if (!fused && (flags & RN_GATE)) return fail(RN_EINVAL, "RN_GATE is only valid for resnorm_fused_fwd");
  if ((flags & RN_BIAS) && !(flags & RN_WEIGHT)) return fail(RN_EINVAL, "RN_BIAS requires RN_WEIGHT");
  if (B < 0 || L < 0) return fail(RN_EINVAL, "negative shape (B=%lld, L=%lld)", (long long)B, (long long)L);
  if (D < 8 || D % 8 != 0) return fail(RN_EINVAL, "D must be a positive multiple of 8 (got %lld)", (long long)D);
  if (D > RN_D_MAX) return fail(RN_EUNSUPPORTED, "D=%lld exceeds RN_D_MAX=%d", (long long)D, RN_D_MAX);
  if (L > 0 && B > ((int64_t)1 << 31) / L) return fail(RN_EUNSUPPORTED, "B*L >= 2^31 rows is not supported");
  if (B * L >= ((int64_t)1 << 31)) return fail(RN_EUNSUPPORTED, "B*L >= 2^31 rows is not supported");
  return RN_OK;
}

// Row operands a kernel holds per row, in units of VPT 16-byte vectors per
// lane (a binary32 weight or bias counts twice).
int row_operands(uint32_t flags, bool fused, int affine_dtype) {
  const int aff = affine_dtype == RN_DTYPE_F32 ? 2 : 1;
  int n = 3;  // x, scale, shift
  if (fused) n += 1 + ((flags & RN_GATE) ? 1 : 0);
  if (flags & RN_WEIGHT) n += aff;
  if (flags & RN_BIAS) n += aff;
  return n;
}

// Tensors streamed through HBM per row: x and y, the residual pair of the
// fused op, and per-row modulation operands.
int hbm_streams(uint32_t flags, bool fused, rn_layout gate_layout, rn_layout ss_layout) {
  int n = 2;
  if (fused) n += 2;
  if (ss_layout.kind == RN_ROW) n += 2;
  if (fused && (flags & RN_GATE) && gate_layout.kind == RN_ROW) n += 1;
  return n;
}

// Rows a multiple of 8 KB apart (D % 4096 == 0): the fused op there takes at
// least this many waves per row.  Measured in one process at D = 4096,
// 220500 rows: two waves x 4 vectors 69.5 % of 8 TB/s against 65.2 % for
// one wave x 8 on torch's back-to-back allocations (every stream in one
// third of physical HBM), but 80.8 % against 83.5 % with the outputs in two
// other thirds.  The rule keeps the gain for ordinary allocations, the
// common case, at a 3 % cost on a planned placement.  (Earlier sweeps had
// seen the one-wave shape switch between two speeds from one process to
// the next; the placement of the tensors in HBM explains that.)
constexpr int kFusedPow2MinWaves = 2;

// Whether every aligned group of k consecutive rows (rows k*m .. k*m + k - 1)
// shares one scale/shift row: always for a broadcast row, for per-frame rows
// when the frame length is a multiple of k (frames tile each batch, so the
// batch length is one too), never for per-row operands.
bool groups_share_ss(rn_layout ss, int64_t L, int k) {
  if (ss.kind == RN_BCAST) return true;
  if (ss.kind != RN_FRAME || ss.frames < 1 || L % ss.frames != 0) return false;
  return (L / ss.frames) % k == 0;
}

// The compiled shape for a problem (see kShapes); -1 if none covers D.
// Waves per row the planner aims for (0: the first compiled shape with W < 10
// that fits the register budget); the measurements behind each rule are
// listed with the shape table.
int preferred_waves(int64_t R, int64_t D, int streams, bool fused, bool one_wave_fits) {
  if (D >= rn::kManyStreamsMinD && streams >= 5) return 10;
  if (D < rn::kSplitMinD) return 0;
  if (R <= rn::kTinyRows && D > 4096 && D <= 5120) return 10;
  if (R <= rn::kSmallRows) return 4;
  if (fused && one_wave_fits && R > 2 * rn::kSmallRows && R <= rn::kFusedOneWaveRows) return 0;
  if (R <= rn::kMidRowsSplit4 && (D >= rn::kManyStreamsMinD || R <= 2 * rn::kSmallRows))
    return D <= 3072 ? 2 : 4;
  if (R <= rn::kMidRows && D >= rn::kManyStreamsMinD) return 2;
  return 0;
}

int shape_for(int64_t R, int64_t L, int64_t D, uint32_t flags, bool fused, int affine_dtype,
              int streams, rn_layout ss_layout) {
  const int64_t nvec = D / 8;
  const int ops = row_operands(flags, fused, affine_dtype);
  const int budget = (!fused && (flags & RN_WEIGHT)) ? rn::kVgprBudgetNormAffine : rn::kVgprBudget;
  // the fused op's one-row shapes with one wave per row stage weight and
  // bias in LDS, so only the row operands take registers
  const int row_ops = row_operands(flags & ~(uint32_t)(RN_WEIGHT | RN_BIAS), fused, affine_dtype);
  auto covers = [&](const rn::Shape& s) { return (int64_t)rn::kWaveSize * s.w * s.vpt >= nvec; };
  auto fits = [&](const rn::Shape& s) {
    if (fused && s.w == 1 && s.k == 1) return s.vpt * row_ops <= budget;
    return s.vpt * ops <= budget;
  };
  // The fused op with rows a multiple of 8 KB apart (D % 4096 == 0) avoids
  // one wave per row (see kFusedPow2MinWaves).
  auto allowed = [&](const rn::Shape& s) {
    return !(fused && D % 4096 == 0 && s.w < kFusedPow2MinWaves);
  };
  if (!fused && (flags & RN_WEIGHT) && R * D >= rn::kMultiRowMinElems) {
    for (int i = 0; i < rn::kNumShapes; ++i) {
      const rn::Shape s = rn::kShapes[i];
      if (s.k > 1 && covers(s) && groups_share_ss(ss_layout, L, s.k)) return i;
    }
  }
  bool one_wave_fits = false;
  for (int i = 0; i < rn::kNumShapes; ++i)
    one_wave_fits = one_wave_fits || (rn::kShapes[i].w == 1 && rn::kShapes[i].k == 1 &&
                                      allowed(rn::kShapes[i]) && covers(rn::kShapes[i]) &&
                                      fits(rn::kShapes[i]));
  const int want = preferred_waves(R, D, streams, fused, one_wave_fits);
  if (want != 0) {
    for (int i = 0; i < rn::kNumShapes; ++i) {
      const rn::Shape s = rn::kShapes[i];
      if (s.k == 1 && s.w == want && allowed(s) && covers(s) && (want == 10 || fits(s)))
        return i;
    }
  }
  // Large problems: the norm-only op without affine streams its rows best
  // with 8 vectors per lane where the first fit would be 6 (2 or 4 waves per
  // row; a sweep of every shape at ~903 M elements, D = 5632-6144 and
  // 10752-12288: 2.3-6.5 % faster, e.g. D = 12288 0.638 -> 0.599 ms;
  // re-measured in one process, D 6144 / 12288: 75.5 / 75.7 % vs 71.5 /
  // 71.3 % of 8 TB/s on back-to-back allocations, 78.3 / 77.8 % vs 75.8 /
  // 75.3 % with the outputs in another third).
  const bool nss_plain = !fused && !(flags & RN_WEIGHT);
  // Large norm-only problems run one-wave shapes of 8 or 10 vectors per lane
  // with 2 rows per workgroup (the twins after the multi-row shapes).
  auto rows2_twin = [&](int i) {
    const rn::Shape s = rn::kShapes[i];
    if (!(nss_plain && s.w == 1 && s.k == 1 && s.vpt >= 8 && R * D >= rn::kMultiRowMinElems)) return i;
    for (int j = 0; j < rn::kNumShapes; ++j) {
      const rn::Shape t = rn::kShapes[j];
      if (t.w == s.w && t.vpt == s.vpt && t.k == 1 && t.rpb == 2) return j;
    }
    return i;
  };
  int fallback = -1;
  for (int i = 0; i < rn::kNumShapes; ++i) {
    const rn::Shape s = rn::kShapes[i];
    if (s.k > 1 || s.w == 10 || !allowed(s) || !covers(s)) continue;
    if (s.w == 1 && s.rpb != 4) continue;  // twins are chosen only through rows2_twin
    if (nss_plain && s.w >= 2 && s.vpt == 6) continue;
    if (fits(s)) return rows2_twin(i);
    if (fallback < 0 || rn::kShapes[fallback].w < s.w) fallback = i;
  }
  return fallback;
}

rn_status validate(const Problem& p) {
  rn_status st = check_shape(p.B, p.L, p.D, p.flags, p.fused);
  if (st != RN_OK) return st;
  const bool want_gate = p.flags & RN_GATE, want_w = p.flags & RN_WEIGHT, want_b = p.flags & RN_BIAS;

  if (!p.y) return fail(RN_EINVAL, "y is NULL");
  if (!p.x) return fail(RN_EINVAL, "x is NULL");
  if (!p.scale) return fail(RN_EINVAL, "scale is NULL");
  if (!p.shift) return fail(RN_EINVAL, "shift is NULL");
  if (p.fused) {
    if (!p.residual) return fail(RN_EINVAL, "residual is NULL");
    if (!p.residual_out) return fail(RN_EINVAL, "residual_out is NULL");
    if (want_gate != (p.gate != nullptr))
      return fail(RN_EINVAL, want_gate ? "RN_GATE set but gate is NULL" : "gate given but RN_GATE not set");
  }
  if (want_w != (p.weight != nullptr))
    return fail(RN_EINVAL, want_w ? "RN_WEIGHT set but weight is NULL" : "weight given but RN_WEIGHT not set");
  if (want_b != (p.bias != nullptr))
    return fail(RN_EINVAL, want_b ? "RN_BIAS set but bias is NULL" : "bias given but RN_BIAS not set");
  if (!std::isfinite(p.eps) || p.eps < 0.f) return fail(RN_EINVAL, "eps must be finite and >= 0 (got %g)", (double)p.eps);
  if (p.affine_dtype != RN_DTYPE_BF16 && p.affine_dtype != RN_DTYPE_F32)
    return fail(RN_EINVAL, "affine_dtype %d is not RN_DTYPE_BF16 or RN_DTYPE_F32", p.affine_dtype);
  if (p.y_dtype != RN_DTYPE_BF16 && p.y_dtype != RN_DTYPE_F32 && p.y_dtype != RN_DTYPE_FP8_E4M3)
    return fail(RN_EINVAL, "y_dtype %d is not RN_DTYPE_BF16, RN_DTYPE_F32 or RN_DTYPE_FP8_E4M3", p.y_dtype);
  if ((p.y_dtype == RN_DTYPE_FP8_E4M3) != (p.y_scale != nullptr))
    return fail(RN_EINVAL, p.y_scale ? "y_scale given but y_dtype is not RN_DTYPE_FP8_E4M3"
                                     : "RN_DTYPE_FP8_E4M3 output needs y_scale");

  if (p.fused && want_gate && (st = check_layout("gate", p.gate_layout, p.L)) != RN_OK) return st;
  if ((st = check_layout("scale/shift", p.ss_layout, p.L)) != RN_OK) return st;

  const void* ptrs[] = {p.y, p.residual_out, p.x, p.residual, p.gate, p.weight, p.bias, p.scale, p.shift};
  const char* names[] = {"y", "residual_out", "x", "residual", "gate", "weight", "bias", "scale", "shift"};
  for (int i = 0; i < 9; ++i)
    if (ptrs[i] && !aligned16(ptrs[i])) return fail(RN_EINVAL, "%s is not 16-byte aligned", names[i]);
  if (p.y_scale && ((uintptr_t)p.y_scale & 3u)) return fail(RN_EINVAL, "y_scale is not 4-byte aligned");

  // Overlap: each output (y, residual_out, y_scale) against every other
  // operand; only exact y == x (bf16 y) and residual_out == residual are
  // allowed.  Inputs may share memory with each other (they are only read).
  const int64_t R = p.B * p.L;
  const uint64_t row = (uint64_t)p.D * 2u;
  const uint64_t y_row = (uint64_t)p.D * (p.y_dtype == RN_DTYPE_F32 ? 4u : p.y_dtype == RN_DTYPE_FP8_E4M3 ? 1u : 2u);
  const uint64_t aff_row = (uint64_t)p.D * (p.affine_dtype == RN_DTYPE_F32 ? 4u : 2u);
  Extent ext[kNumOperands];
  int n = 0, n_out = 0;
  auto add = [&](int id, const void* ptr, int64_t rows, uint64_t row_bytes) {
    if (ptr && rows > 0) ext[n++] = Extent{id, (uintptr_t)ptr, (uintptr_t)ptr + (uintptr_t)(rows * row_bytes)};
  };
  add(kY, p.y, R, y_row);  // the outputs first
  if (p.fused) add(kResidualOut, p.residual_out, R, row);
  add(kYScale, p.y_scale, R, 4);
  n_out = n;
  add(kX, p.x, R, row);
  if (p.fused) add(kResidual, p.residual, R, row);
  if (p.fused && want_gate) add(kGate, p.gate, layout_rows(p.gate_layout, p.B, p.L), row);
  add(kWeight, p.weight, 1, aff_row);
  add(kBias, p.bias, 1, aff_row);
  add(kScale, p.scale, layout_rows(p.ss_layout, p.B, p.L), row);
  add(kShift, p.shift, layout_rows(p.ss_layout, p.B, p.L), row);
  for (int i = 0; i < n_out; ++i) {
    const Extent& a = ext[i];
    // the pair of a that may alias it exactly
    const int alias = a.id == kY ? kX : a.id == kResidualOut ? kResidual : -1;
    for (int j = i + 1; j < n; ++j) {
      const Extent& b = ext[j];
      if (a.lo >= b.hi || b.lo >= a.hi) continue;
      if (b.id == alias && a.lo == b.lo && a.hi == b.hi) continue;
      return fail(RN_EINVAL, "%s overlaps %s", kOperandName[a.id], kOperandName[b.id]);
    }
  }
  return RN_OK;
}

rn::KernelFn pick_kernel(const Problem& p, int vi) {
  const bool f32 = p.affine_dtype == RN_DTYPE_F32;
  const int aff = (p.flags & RN_BIAS)     ? (f32 ? rn::kAffWB32 : rn::kAffWB16)
                  : (p.flags & RN_WEIGHT) ? (f32 ? rn::kAffW32 : rn::kAffW16)
                                          : rn::kAffNone;
  const bool rms = p.flags & RN_RMS;
  const int out = p.y_dtype == RN_DTYPE_FP8_E4M3 ? rn::kOutFp8
                  : p.y_dtype == RN_DTYPE_F32     ? rn::kOutF32
                                                  : rn::kOutBf16;
  if (p.fused) return rn::fused_kernel(rms, out, p.flags & RN_GATE, aff, vi);
  return rn::nss_kernel(rms, out, aff, vi);
}

uint32_t tokens_per_frame(rn_layout lay, int64_t L) {
  return lay.kind == RN_FRAME ? (uint32_t)(L / lay.frames) : 1u;
}

bool same_layout(rn_layout a, rn_layout b) { return a.kind == b.kind && a.frames == b.frames; }

// Field-wise equality of two problems (every field the validation and the
// launch plan read).
bool same_problem(const Problem& a, const Problem& b) {
  return a.fused == b.fused && a.affine_dtype == b.affine_dtype && a.y_dtype == b.y_dtype &&
         a.y_scale == b.y_scale && a.y == b.y && a.residual_out == b.residual_out && a.x == b.x &&
         a.residual == b.residual && a.gate == b.gate && a.weight == b.weight && a.bias == b.bias &&
         a.scale == b.scale && a.shift == b.shift && a.B == b.B && a.L == b.L && a.D == b.D &&
         a.flags == b.flags && same_layout(a.gate_layout, b.gate_layout) &&
         same_layout(a.ss_layout, b.ss_layout) &&
         __builtin_memcmp(&a.eps, &b.eps, sizeof a.eps) == 0;
}

// A validated launch: kernel, grid, workgroup size and arguments.
struct Launch {
  rn::KernelFn fn;
  dim3 grid, block;
  rn::RowArgs a;
};

// Validation and planning are pure functions of the arguments, so the last
// validated problem of each thread is kept with its launch: a call that
// repeats it exactly (the same buffers and sizes, as a denoising loop makes
// every step) goes straight to the launch.  Only successful validations are
// kept; a rejected call never reaches the cache.
struct LastLaunch {
  bool valid = false;
  Problem p;
  Launch l;
};
thread_local LastLaunch g_last;

// Validate and plan; RN_OK with l.fn == nullptr for an empty problem.
rn_status plan_launch(const Problem& p, Launch& l) {
  rn_status st = validate(p);
  if (st != RN_OK) return st;
  const int64_t R = p.B * p.L;
  l.fn = nullptr;
  if (R == 0) return RN_OK;
  const int vi = shape_for(R, p.L, p.D, p.flags, p.fused, p.affine_dtype,
                           hbm_streams(p.flags, p.fused, p.gate_layout, p.ss_layout), p.ss_layout);
  rn::KernelFn fn = vi < 0 ? nullptr : pick_kernel(p, vi);
  if (!fn) return fail(RN_EUNSUPPORTED, "no compiled kernel for D=%lld flags=0x%x", (long long)p.D, p.flags);

  rn::RowArgs& a = l.a;
  a.x = p.x;
  a.residual = p.residual;
  a.gate = p.gate;
  a.weight = p.weight;
  a.bias = p.bias;
  a.scale = p.scale;
  a.shift = p.shift;
  a.y = p.y;
  a.residual_out = p.residual_out;
  a.y_scale = p.y_scale;
  a.rows = (uint32_t)R;
  a.L = (uint32_t)p.L;
  a.d = (uint32_t)p.D;
  a.nvec = (uint32_t)(p.D / 8);
  a.eps = p.eps;
  // The gate's layout is validated, and used, only when the gate is flagged;
  // otherwise it is ignored (any value).
  const rn_layout gl = (p.fused && (p.flags & RN_GATE)) ? p.gate_layout : rn_layout{RN_BCAST, 0};
  a.gate_kind = gl.kind;
  a.gate_frames = (uint32_t)(gl.kind == RN_FRAME ? gl.frames : 0);
  a.gate_tokens_per_frame = tokens_per_frame(gl, p.L);
  a.ss_kind = p.ss_layout.kind;
  a.ss_frames = (uint32_t)(p.ss_layout.kind == RN_FRAME ? p.ss_layout.frames : 0);
  a.ss_tokens_per_frame = tokens_per_frame(p.ss_layout, p.L);

  const rn::Shape shape = rn::kShapes[vi];
  const int64_t rows_per_block = (int64_t)shape.rpb * shape.k;
  const int64_t blocks = (R + rows_per_block - 1) / rows_per_block;
  const int64_t threads = (int64_t)rn::kWaveSize * shape.w * shape.rpb;
  // A dispatch counts work-items per grid dimension in 32 bits: beyond that
  // the workgroups continue in y (the kernel numbers them x-fastest; the
  // surplus of the last y row finds no row and exits).
  const int64_t max_x = (int64_t)UINT32_MAX / threads;
  const int64_t gx = blocks < max_x ? blocks : max_x;
  const int64_t gy = (blocks + gx - 1) / gx;
  l.fn = fn;
  l.grid = dim3((uint32_t)gx, (uint32_t)gy);
  l.block = dim3((uint32_t)threads);
  return RN_OK;
}

rn_status run(const Problem& p, void* stream) {
  g_err[0] = '\0';
  if (!(g_last.valid && same_problem(g_last.p, p))) {
    g_last.valid = false;
    Launch l;
    const rn_status st = plan_launch(p, l);
    if (st != RN_OK) return st;
    g_last.p = p;
    g_last.l = l;
    g_last.valid = true;
  }
  Launch& l = g_last.l;
  if (!l.fn) return RN_OK;  // empty problem: nothing to enqueue
  void* args[] = {&l.a};
  hipError_t e = hipLaunchKernel((const void*)l.fn, l.grid, l.block, args, 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RN_ELAUNCH, "hipLaunchKernel failed: %s", hipGetErrorString(e));
  return RN_OK;
}

}  // namespace

extern "C" {

static void apply_ext(Problem& p, const rn_ext* ext) {
  p.affine_dtype = ext ? ext->affine_dtype : RN_DTYPE_BF16;
  p.y_dtype = ext ? ext->y_dtype : RN_DTYPE_BF16;
  p.y_scale = ext ? (float*)ext->y_scale : nullptr;
}

rn_status resnorm_fused_fwd_ex(void* y, void* residual_out, const void* x, const void* residual,
                               const void* gate, const void* weight, const void* bias,
                               const void* scale, const void* shift, int64_t B, int64_t L,
                               int64_t D, uint32_t flags, rn_layout gate_layout,
                               rn_layout ss_layout, float eps, const rn_ext* ext, void* stream) {
  Problem p{};
  p.fused = true;
  p.y = y;
  p.residual_out = residual_out;
  p.x = x;
  p.residual = residual;
  p.gate = gate;
  p.weight = weight;
  p.bias = bias;
  p.scale = scale;
  p.shift = shift;
  p.B = B;
  p.L = L;
  p.D = D;
  p.flags = flags;
  p.gate_layout = gate_layout;
  p.ss_layout = ss_layout;
  p.eps = eps;
  apply_ext(p, ext);
  return run(p, stream);
}

rn_status norm_scale_shift_fwd_ex(void* y, const void* x, const void* weight, const void* bias,
                                  const void* scale, const void* shift, int64_t B, int64_t L,
                                  int64_t D, uint32_t flags, rn_layout ss_layout, float eps,
                                  const rn_ext* ext, void* stream) {
  Problem p{};
  p.fused = false;
  p.y = y;
  p.x = x;
  p.weight = weight;
  p.bias = bias;
  p.scale = scale;
  p.shift = shift;
  p.B = B;
  p.L = L;
  p.D = D;
  p.flags = flags;
  p.gate_layout = rn_layout{RN_BCAST, 0};
  p.ss_layout = ss_layout;
  p.eps = eps;
  apply_ext(p, ext);
  return run(p, stream);
}

rn_status resnorm_fused_fwd(void* y, void* residual_out, const void* x, const void* residual,
                            const void* gate, const void* weight, const void* bias, const void* scale,
                            const void* shift, int64_t B, int64_t L, int64_t D, uint32_t flags,
                            rn_layout gate_layout, rn_layout ss_layout, float eps, void* stream) {
  return resnorm_fused_fwd_ex(y, residual_out, x, residual, gate, weight, bias, scale, shift, B, L, D,
                              flags, gate_layout, ss_layout, eps, nullptr, stream);
}

rn_status norm_scale_shift_fwd(void* y, const void* x, const void* weight, const void* bias,
                               const void* scale, const void* shift, int64_t B, int64_t L, int64_t D,
                               uint32_t flags, rn_layout ss_layout, float eps, void* stream) {
  return norm_scale_shift_fwd_ex(y, x, weight, bias, scale, shift, B, L, D, flags, ss_layout, eps,
                                 nullptr, stream);
}

const char* rn_last_error(void) { return g_err; }

rn_status rn_describe_launch_ex(int64_t B, int64_t L, int64_t D, uint32_t flags, int32_t fused,
                                rn_layout gate_layout, rn_layout ss_layout, const rn_ext* ext,
                                rn_launch_info* info) {
  g_err[0] = '\0';
  if (!info) return fail(RN_EINVAL, "info is NULL");
  rn_status st = check_shape(B, L, D, flags, fused != 0);
  if (st != RN_OK) return st;
  const int affine_dtype = ext ? ext->affine_dtype : RN_DTYPE_BF16;
  if (affine_dtype != RN_DTYPE_BF16 && affine_dtype != RN_DTYPE_F32)
    return fail(RN_EINVAL, "affine_dtype %d is not RN_DTYPE_BF16 or RN_DTYPE_F32", affine_dtype);
  // the layouts a launch would refuse are refused here too
  if (fused && (flags & RN_GATE) && (st = check_layout("gate", gate_layout, L)) != RN_OK) return st;
  if ((st = check_layout("scale/shift", ss_layout, L)) != RN_OK) return st;
  const int vi = shape_for(B * L, L, D, flags, fused != 0, affine_dtype,
                           hbm_streams(flags, fused != 0, gate_layout, ss_layout), ss_layout);
  if (vi < 0) return fail(RN_EUNSUPPORTED, "no compiled shape covers D=%lld", (long long)D);
  const rn::Shape s = rn::kShapes[vi];
  info->vec_per_lane = s.vpt;
  info->waves_per_row = s.w;
  info->waves_per_block = s.w * s.rpb;
  info->rows_per_block = s.rpb * s.k;
  info->block_threads = rn::kWaveSize * s.w * s.rpb;
  info->grid_blocks = (B * L + info->rows_per_block - 1) / info->rows_per_block;
  info->rows_per_wave = s.k;
  return RN_OK;
}

rn_status rn_describe_launch(int64_t B, int64_t L, int64_t D, uint32_t flags, int32_t fused,
                             rn_layout gate_layout, rn_layout ss_layout, rn_launch_info* info) {
  return rn_describe_launch_ex(B, L, D, flags, fused, gate_layout, ss_layout, nullptr, info);
}

const char* rn_version(void) { return "resnorm 0.3.0 gfx950"; }

}  // extern "C"
