// The C ABI of libtwell.so (declared in include/twell.h): argument checks,
// workspace carving and the launch sequence of each entry point.  All work
// is enqueued on the caller's stream; nothing here synchronises the host.
#include "../../include/twell.h"
#include "kernels.h"

#include <mutex>

#define TWELL_EXPORT extern "C" __attribute__((visibility("default")))

namespace twell {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int32_t dtype) { return dtype == TWELL_F32 ? 4 : 2; }

// Geometry checks shared by every entry point.  `need_model` adds the
// d_model requirements (not used by pack / unpack).
int check_shape(const twell_shape* s, bool need_model) {
  if (s == nullptr) return TWELL_ERR_INVALID_ARG;
  if (s->n_rows < 0 || s->n_rows > INT32_MAX) return TWELL_ERR_INVALID_ARG;
  if (s->dtype != TWELL_F32 && s->dtype != TWELL_BF16) return TWELL_ERR_INVALID_ARG;
  if (s->reserved != 0) return TWELL_ERR_INVALID_ARG;
  if (s->d_ff <= 0 || s->tile <= 0 || s->tile > 256 || s->d_ff % s->tile != 0)
    return TWELL_ERR_INVALID_ARG;
  if (s->capacity < 1 || s->capacity > s->tile || s->capacity > 255) return TWELL_ERR_INVALID_ARG;
  if (need_model && (s->d_model <= 0 || s->d_model % 8 != 0)) return TWELL_ERR_INVALID_ARG;
  if (s->tile != 64 && s->tile != 128 && s->tile != 256) return TWELL_ERR_UNSUPPORTED;
  return TWELL_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ELL rows: one tile spanning the row (tile == d_ff), capacity = width.
int check_ell_shape(const twell_shape* s, bool need_model) {
  if (s == nullptr) return TWELL_ERR_INVALID_ARG;
  if (s->n_rows < 0 || s->n_rows > INT32_MAX) return TWELL_ERR_INVALID_ARG;
  if (s->dtype != TWELL_F32 && s->dtype != TWELL_BF16) return TWELL_ERR_INVALID_ARG;
  if (s->reserved != 0) return TWELL_ERR_INVALID_ARG;
  if (s->d_ff <= 0 || s->d_ff > 65536 || s->d_ff % 8 != 0 || s->tile != s->d_ff)
    return TWELL_ERR_INVALID_ARG;
  if (s->capacity < 1 || s->capacity > s->d_ff || s->capacity > 65535) return TWELL_ERR_INVALID_ARG;
  if (need_model && (s->d_model <= 0 || s->d_model % 8 != 0)) return TWELL_ERR_INVALID_ARG;
  return TWELL_OK;
}

int check_ell(const twell_ell* e, int64_t n_rows) {
  if (e == nullptr || e->n_dense == nullptr || e->dense_capacity < 0) return TWELL_ERR_INVALID_ARG;
  if (!aligned16(e->values) || !aligned16(e->columns) || !aligned16(e->counts) ||
      !aligned16(e->dense_rows) || !aligned16(e->dense_values))
    return TWELL_ERR_INVALID_ARG;
  if (n_rows > 0 && (e->values == nullptr || e->columns == nullptr || e->counts == nullptr))
    return TWELL_ERR_INVALID_ARG;
  if (e->dense_capacity > 0 && (e->dense_rows == nullptr || e->dense_values == nullptr))
    return TWELL_ERR_INVALID_ARG;
  return TWELL_OK;
}

int check_hybrid(const twell_hybrid* h, int64_t n_rows) {
  if (h == nullptr || h->n_dense == nullptr || h->dense_capacity < 0) return TWELL_ERR_INVALID_ARG;
  if (!aligned16(h->values) || !aligned16(h->indices) || !aligned16(h->counts) ||
      !aligned16(h->dense_rows) || !aligned16(h->dense_values))
    return TWELL_ERR_INVALID_ARG;
  if (n_rows > 0 && (h->values == nullptr || h->indices == nullptr || h->counts == nullptr))
    return TWELL_ERR_INVALID_ARG;
  if (h->dense_capacity > 0 && (h->dense_rows == nullptr || h->dense_values == nullptr))
    return TWELL_ERR_INVALID_ARG;
  return TWELL_OK;
}

Geometry geometry(const twell_shape* s) {
  Geometry g;
  g.n_rows = s->n_rows;
  g.d_model = s->d_model;
  g.d_ff = s->d_ff;
  g.tile = s->tile;
  g.capacity = s->capacity;
  g.n_tiles = s->d_ff / s->tile;
  return g;
}

struct PackWorkspace {
  RouteBufs route;
  void* spill;
  float* skinny;  // split-K partial sums for batches of few rows, or nullptr
};

// Workspace: flags [N][nt] u8 | row_dense [N] u8 | row_map [N] i32 |
// sparse_rows [N] i32 | n_sparse i32 | (forward only) spill [N][d_ff] dtype |
// (forward only, at most 64 rows) split-K partial sums, each part 256-byte
// aligned.
size_t pack_ws_bytes(const twell_shape* s) {
  const size_t n = static_cast<size_t>(s->n_rows);
  return align_up(n * static_cast<size_t>(s->d_ff / s->tile)) + align_up(n) +
         2 * align_up(n * sizeof(int32_t)) + align_up(sizeof(int32_t));
}

size_t fwd_ws_bytes(const twell_shape* s) {
  const size_t n = static_cast<size_t>(s->n_rows);
  return pack_ws_bytes(s) + align_up(n * static_cast<size_t>(s->d_ff) * elem_bytes(s->dtype)) +
         align_up(skinny_ws_bytes(geometry(s)));
}

// twell_spmm's optional workspace: the split-K kernels' partial sums for at
// most 64 rows; for bf16 beyond that, room for 32 K slices of every row, at
// most 32 MiB (the 128 x 128 tile kernel's 512 workgroups never hold more:
// slices x live tiles <= 512, 64 KiB of partial sums each).
size_t spmm_ws_bytes(const twell_shape* s) {
  const Geometry g = geometry(s);
  size_t b = skinny_ws_bytes(g);
  if (s->dtype == TWELL_BF16 && b == 0) {
    const size_t all = size_t{32} * static_cast<size_t>(s->n_rows) *
                       static_cast<size_t>(s->d_model) * sizeof(float);
    b = align_up(all < (size_t{32} << 20) ? all : (size_t{32} << 20));
  }
  return b;
}

// Floats that fit in the forward's spill area [N][d_ff] of dtype.
int64_t spill_floats(const twell_shape* s) {
  return static_cast<int64_t>(s->n_rows) * s->d_ff * elem_bytes(s->dtype) / 4;
}

PackWorkspace carve(const twell_shape* s, void* ws, bool with_spill) {
  PackWorkspace w;
  const size_t n = static_cast<size_t>(s->n_rows);
  uint8_t* p = static_cast<uint8_t*>(ws);
  w.route.flags = p;
  p += align_up(n * static_cast<size_t>(s->d_ff / s->tile));
  w.route.row_dense = p;
  p += align_up(n);
  w.route.row_map = reinterpret_cast<int32_t*>(p);
  p += align_up(n * sizeof(int32_t));
  w.route.sparse_rows = reinterpret_cast<int32_t*>(p);
  p += align_up(n * sizeof(int32_t));
  w.route.n_sparse = reinterpret_cast<int32_t*>(p);
  p += align_up(sizeof(int32_t));
  w.spill = with_spill ? p : nullptr;
  w.skinny = nullptr;
  if (with_spill) {
    p += align_up(n * static_cast<size_t>(s->d_ff) * elem_bytes(s->dtype));
    if (skinny_ws_bytes(geometry(s)) > 0) w.skinny = reinterpret_cast<float*>(p);
  }
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TWELL_OK : TWELL_ERR_HIP; }

#define TWELL_TRY(expr)                          \
  do {                                           \
    const hipError_t e_ = (expr);                \
    if (e_ != hipSuccess) return TWELL_ERR_HIP;  \
  } while (0)

// Steps 2-4 of the forward pass once the pack step has run: route, build
// the dense rows, sparse product, dense fallback.
// With `sp` (build_takes_spmm held), the build also runs the sparse product.
int route_and_materialize(const Geometry& g, int eb, const PackWorkspace& w, const void* full_src,
                          const twell_hybrid* hy, int32_t* d_status, hipStream_t st,
                          const BuildSpmm* sp = nullptr) {
  if (route_mode(g) != 0) {
    // the dense-row build routes the rows itself: no scan kernel
    TWELL_TRY(launch_route_materialize(g, eb, w.route, w.spill, full_src, hy->values,
                                       hy->indices, hy->counts, hy->dense_rows, hy->dense_values,
                                       hy->dense_capacity, hy->n_dense, d_status, st, sp));
    return TWELL_OK;
  }
  if (sp != nullptr) return TWELL_ERR_INVALID_ARG;
  TWELL_TRY(launch_route_scan(g, w.route, hy->dense_rows, hy->dense_capacity, hy->n_dense,
                              d_status, st));
  TWELL_TRY(launch_materialize(g, eb, w.route.row_map, w.route.flags, w.spill, full_src, hy->values,
                               hy->indices, hy->counts, hy->dense_values, hy->dense_capacity, st));
  return TWELL_OK;
}

}  // namespace
}  // namespace twell

using namespace twell;

TWELL_EXPORT int twell_version(void) { return TWELL_VERSION; }

TWELL_EXPORT const char* twell_status_string(int status) {
  switch (status) {
    case TWELL_OK: return "ok";
    case TWELL_ERR_INVALID_ARG: return "invalid argument";
    case TWELL_ERR_UNSUPPORTED: return "unsupported geometry";
    case TWELL_ERR_WORKSPACE: return "workspace too small";
    case TWELL_ERR_HIP: return "HIP launch failed";
    case TWELL_ERR_DENSE_CAPACITY: return "more dense rows than dense_capacity";
    case TWELL_ERR_SCRATCH_LIMIT: return "shape needs more than the fixed device scratch";
    default: return "unknown status";
  }
}

TWELL_EXPORT size_t ffn_sparse_workspace_size(const twell_shape* shape) {
  if (check_shape(shape, true) != TWELL_OK) return 0;
  return fwd_ws_bytes(shape);
}

TWELL_EXPORT size_t twell_pack_workspace_size(const twell_shape* shape) {
  if (check_shape(shape, false) != TWELL_OK) return 0;
  return pack_ws_bytes(shape);
}

namespace twell {
namespace {

// The forward pass; `ev`, when given, holds five events recorded on the
// stream before step 1 and after each of steps 1-4 (which then run in
// order on the stream).
// The gated layer's up branch: step 1 then runs on the gate's weights (the
// x, w_up_t, b_up arguments), and the up branch is applied at the gate's
// non-zeros between steps 2 and 3.
struct GateArgs {
  const void* w_up_t;
  const float* b_up;
};

int forward_impl(const twell_shape* shape, const void* x, const void* w_up_t, const float* b_up,
                 const void* w_down, void* y, const twell_hybrid* h_out, void* h_dense_debug,
                 void* workspace, size_t workspace_bytes, int32_t* d_status, void* stream,
                 void* const* ev, const GateArgs* gate = nullptr) {
  int rc = check_shape(shape, true);
  if (rc != TWELL_OK) return rc;
  const Geometry g = geometry(shape);
  if ((rc = check_hybrid(h_out, g.n_rows)) != TWELL_OK) return rc;
  if (g.n_rows > 0 && (x == nullptr || w_up_t == nullptr || b_up == nullptr || w_down == nullptr ||
                       y == nullptr))
    return TWELL_ERR_INVALID_ARG;
  if (workspace == nullptr) return TWELL_ERR_INVALID_ARG;  // the routing writes it even for 0 rows
  if (!aligned16(x) || !aligned16(w_up_t) || !aligned16(w_down) || !aligned16(y) ||
      !aligned16(h_dense_debug) || !aligned16(workspace))
    return TWELL_ERR_INVALID_ARG;
  if (ev != nullptr) {
    for (int i = 0; i < 5; ++i)
      if (ev[i] == nullptr) return TWELL_ERR_INVALID_ARG;
  }
  if (workspace_bytes < fwd_ws_bytes(shape)) return TWELL_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    return ev != nullptr ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), st) : hipSuccess;
  };
  const int eb = elem_bytes(shape->dtype);
  const PackWorkspace w = carve(shape, workspace, true);

  TWELL_TRY(mark(0));
  // 1. up-projection + bias + ReLU with the TwELL pack in its epilogue
  PackOut po{h_out->values, h_out->indices, h_out->counts, w.route.flags, w.spill, h_dense_debug,
             w.skinny};
  if (g.n_rows > 0) {
    if (eb == 2)
      TWELL_TRY(launch_up_pack_bf16(g, static_cast<const uint16_t*>(x),
                                    static_cast<const uint16_t*>(w_up_t), b_up, po, st));
    else
      TWELL_TRY(launch_up_pack_f32(g, static_cast<const float*>(x),
                                   static_cast<const float*>(w_up_t), b_up, po, st));
  }
  TWELL_TRY(mark(1));
  // 2. route rows, build dense rows from the TwELL slots + spilled tiles; for
  // float32 batches of at most 64 rows (plain call) the build's sparse-row
  // workgroups also run step 3 for their rows
  const bool build_spmm = ev == nullptr && gate == nullptr && g.n_rows > 0 && build_takes_spmm(g, eb);
  const BuildSpmm bsp{w_down, y};
  if ((rc = route_and_materialize(g, eb, w, nullptr, h_out, d_status, st,
                                  build_spmm ? &bsp : nullptr)) != TWELL_OK)
    return rc;
  if (gate != nullptr) {
    // the gated layer: h = gate * (x W_up + b_up) at the gate's non-zeros
    const GateHybrid gh{h_out->values,       h_out->indices, h_out->counts,
                        h_out->dense_rows,   h_out->dense_values, h_out->n_dense,
                        h_out->dense_capacity, w.route.sparse_rows, w.route.n_sparse};
    TWELL_TRY(launch_gate_up(g, eb, gh, x, gate->w_up_t, gate->b_up, st));
  }
  TWELL_TRY(mark(2));
  // 3. sparse down-projection of the TwELL rows and 4. dense fallback for the
  // dense rows, one after the other on the caller's stream (they write
  // disjoint rows of y).
  if (g.n_rows > 0) {
    // batches of at most 64 bf16 rows (plain call): the sparse product runs as
    // extra workgroups of the fallback's split-K launch, inside its weight stream
    const bool merged = ev == nullptr && eb == 2 && w.skinny != nullptr && fallback_takes_spmm(g);
    if (merged) {
      const SpmmRows sr{static_cast<const uint16_t*>(h_out->values), h_out->indices,
                        h_out->counts, w.route.sparse_rows, w.route.n_sparse};
      TWELL_TRY(launch_fallback_bf16_with_spmm(
          g, static_cast<const uint16_t*>(h_out->dense_values), h_out->dense_rows, h_out->n_dense,
          h_out->dense_capacity, static_cast<const uint16_t*>(w_down), static_cast<uint16_t*>(y),
          st, w.skinny, sr));
    } else if (!build_spmm) {
      TWELL_TRY(launch_spmm_sparse(g, eb, h_out->values, h_out->indices, h_out->counts,
                                   w.route.sparse_rows, w.route.n_sparse, nullptr, w_down, y, st));
    }
    TWELL_TRY(mark(3));
    if (merged) {
      // done above
    } else if (eb == 2)
      // the spill area has been read by step 2: step 4 may keep partial sums there
      TWELL_TRY(launch_fallback_bf16(g, static_cast<const uint16_t*>(h_out->dense_values),
                                     h_out->dense_rows, h_out->n_dense, h_out->dense_capacity,
                                     static_cast<const uint16_t*>(w_down),
                                     static_cast<uint16_t*>(y), st, w.skinny,
                                     static_cast<float*>(w.spill), spill_floats(shape)));
    else
      TWELL_TRY(launch_fallback_f32(g, static_cast<const float*>(h_out->dense_values),
                                    h_out->dense_rows, h_out->n_dense, h_out->dense_capacity,
                                    static_cast<const float*>(w_down), static_cast<float*>(y),
                                    st, w.skinny));
  } else {
    TWELL_TRY(mark(3));
  }
  TWELL_TRY(mark(4));
  return TWELL_OK;
}

}  // namespace
}  // namespace twell

TWELL_EXPORT int ffn_sparse_gated_forward(const twell_shape* shape, const void* x,
                                          const void* w_gate_t, const float* b_gate,
                                          const void* w_up_t, const float* b_up,
                                          const void* w_down, void* y, const twell_hybrid* h_out,
                                          void* workspace, size_t workspace_bytes,
                                          int32_t* d_status, void* stream) {
  const int rc = check_shape(shape, true);
  if (rc != TWELL_OK) return rc;
  if (shape->n_rows > 0 && (w_up_t == nullptr || b_up == nullptr)) return TWELL_ERR_INVALID_ARG;
  if (!aligned16(w_up_t)) return TWELL_ERR_INVALID_ARG;
  if (!gate_supported(geometry(shape), elem_bytes(shape->dtype))) return TWELL_ERR_UNSUPPORTED;
  const GateArgs gate{w_up_t, b_up};
  return forward_impl(shape, x, w_gate_t, b_gate, w_down, y, h_out, nullptr, workspace,
                      workspace_bytes, d_status, stream, nullptr, &gate);
}

TWELL_EXPORT int ffn_sparse_forward(const twell_shape* shape, const void* x, const void* w_up_t,
                                    const float* b_up, const void* w_down, void* y,
                                    const twell_hybrid* h_out, void* h_dense_debug,
                                    void* workspace, size_t workspace_bytes, int32_t* d_status,
                                    void* stream) {
  return forward_impl(shape, x, w_up_t, b_up, w_down, y, h_out, h_dense_debug, workspace,
                      workspace_bytes, d_status, stream, nullptr);
}

TWELL_EXPORT int ffn_sparse_forward_events(const twell_shape* shape, const void* x,
                                           const void* w_up_t, const float* b_up,
                                           const void* w_down, void* y, const twell_hybrid* h_out,
                                           void* h_dense_debug, void* workspace,
                                           size_t workspace_bytes, int32_t* d_status, void* stream,
                                           void* const* stage_events) {
  if (stage_events == nullptr) return TWELL_ERR_INVALID_ARG;
  return forward_impl(shape, x, w_up_t, b_up, w_down, y, h_out, h_dense_debug, workspace,
                      workspace_bytes, d_status, stream, stage_events);
}

namespace twell {
namespace {

int pack_impl(const twell_shape* shape, const void* h, const twell_hybrid* out, void* workspace,
              size_t workspace_bytes, int32_t* d_status, void* stream) {
  int rc = check_shape(shape, false);
  if (rc != TWELL_OK) return rc;
  const Geometry g = geometry(shape);
  if ((rc = check_hybrid(out, g.n_rows)) != TWELL_OK) return rc;
  if ((g.n_rows > 0 && h == nullptr) || workspace == nullptr) return TWELL_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(workspace)) return TWELL_ERR_INVALID_ARG;
  if (workspace_bytes < pack_ws_bytes(shape)) return TWELL_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int eb = elem_bytes(shape->dtype);
  const PackWorkspace w = carve(shape, workspace, false);
  PackOut po{out->values, out->indices, out->counts, w.route.flags, nullptr, nullptr, nullptr};
  TWELL_TRY(launch_pack_tiles(g, h, eb, po, st));
  return route_and_materialize(g, eb, w, h, out, d_status, st);
}

// ---- twell_pack_noalloc: the workspace is this fixed device array, one copy
// per GPU.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies get the address that hipGetSymbolAddress
// returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = TWELL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchAddr {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
};
ScratchAddr g_scratch[kMaxDevices];

// The current device's copy of `scratch`, or nullptr (with *err set).
void* scratch_address(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  ScratchAddr* a = &g_scratch[dev];
  std::call_once(a->once, [a] {
    a->err = hipGetSymbolAddress(&a->ptr, HIP_SYMBOL(scratch));
    if (a->err == hipSuccess && a->ptr == nullptr) a->err = hipErrorInvalidSymbol;
  });
  *err = a->err;
  return a->err == hipSuccess ? a->ptr : nullptr;
}

}  // namespace
}  // namespace twell

TWELL_EXPORT int twell_pack(const twell_shape* shape, const void* h, const twell_hybrid* out,
                            void* workspace, size_t workspace_bytes, int32_t* d_status,
                            void* stream) {
  return pack_impl(shape, h, out, workspace, workspace_bytes, d_status, stream);
}

TWELL_EXPORT int twell_pack_noalloc(const twell_shape* shape, const void* h,
                                    const twell_hybrid* out, int32_t* d_status, void* stream) {
  const int rc = check_shape(shape, false);
  if (rc != TWELL_OK) return rc;
  const size_t need = pack_ws_bytes(shape);
  if (need > kScratchBytes) return TWELL_ERR_SCRATCH_LIMIT;
  hipError_t e = hipSuccess;
  void* ws = scratch_address(&e);
  if (ws == nullptr) return TWELL_ERR_HIP;
  return pack_impl(shape, h, out, ws, kScratchBytes, d_status, stream);
}

TWELL_EXPORT int twell_unpack(const twell_shape* shape, const twell_hybrid* in, void* h,
                              void* stream) {
  int rc = check_shape(shape, false);
  if (rc != TWELL_OK) return rc;
  const Geometry g = geometry(shape);
  if ((rc = check_hybrid(in, g.n_rows)) != TWELL_OK) return rc;
  if (g.n_rows > 0 && h == nullptr) return TWELL_ERR_INVALID_ARG;
  if (!aligned16(h)) return TWELL_ERR_INVALID_ARG;
  return hip_status(launch_unpack(g, elem_bytes(shape->dtype), in->values, in->indices, in->counts,
                                  in->dense_rows, in->dense_values, in->n_dense,
                                  in->dense_capacity, h, static_cast<hipStream_t>(stream)));
}

TWELL_EXPORT size_t twell_spmm_workspace_size(const twell_shape* shape) {
  if (check_shape(shape, true) != TWELL_OK) return 0;
  return spmm_ws_bytes(shape);
}

TWELL_EXPORT int twell_spmm(const twell_shape* shape, const twell_hybrid* in, const void* w_down,
                            void* y, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape, true);
  if (rc != TWELL_OK) return rc;
  const Geometry g = geometry(shape);
  if ((rc = check_hybrid(in, g.n_rows)) != TWELL_OK) return rc;
  if (g.n_rows > 0 && (w_down == nullptr || y == nullptr)) return TWELL_ERR_INVALID_ARG;
  if (!aligned16(w_down) || !aligned16(y) || !aligned16(workspace)) return TWELL_ERR_INVALID_ARG;
  if (workspace != nullptr && workspace_bytes < spmm_ws_bytes(shape)) return TWELL_ERR_WORKSPACE;
  if (g.n_rows == 0) return TWELL_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int eb = elem_bytes(shape->dtype);
  // the TwELL rows (a row listed among the stored dense rows is skipped) ...
  const DenseSkip skip{in->dense_rows, in->n_dense, in->dense_capacity};
  TWELL_TRY(launch_spmm_sparse(g, eb, in->values, in->indices, in->counts, nullptr, nullptr,
                               in->dense_capacity > 0 ? &skip : nullptr, w_down, y, st));
  // ... and the stored dense rows by the dense fallback GEMM, splitting K
  // over the workspace's partial sums when there is one
  float* ws = workspace != nullptr && spmm_ws_bytes(shape) > 0 ? static_cast<float*>(workspace)
                                                              : nullptr;
  float* skinny = ws != nullptr && skinny_ws_bytes(g) > 0 ? ws : nullptr;
  if (eb == 2)
    TWELL_TRY(launch_fallback_bf16(g, static_cast<const uint16_t*>(in->dense_values),
                                   in->dense_rows, in->n_dense, in->dense_capacity,
                                   static_cast<const uint16_t*>(w_down), static_cast<uint16_t*>(y),
                                   st, skinny, ws,
                                   ws != nullptr ? static_cast<int64_t>(workspace_bytes / 4) : 0));
  else
    TWELL_TRY(launch_fallback_f32(g, static_cast<const float*>(in->dense_values), in->dense_rows,
                                  in->n_dense, in->dense_capacity,
                                  static_cast<const float*>(w_down), static_cast<float*>(y), st,
                                  skinny));
  return TWELL_OK;
}

// ------------------------------------------------------------------ ELL rows
TWELL_EXPORT size_t ell_pack_workspace_size(const twell_shape* shape) {
  if (check_ell_shape(shape, false) != TWELL_OK) return 0;
  return pack_ws_bytes(shape);  // one "tile" per row: one flag per row
}

TWELL_EXPORT int ell_pack(const twell_shape* shape, const void* h, const twell_ell* out,
                          void* workspace, size_t workspace_bytes, int32_t* d_status,
                          void* stream) {
  int rc = check_ell_shape(shape, false);
  if (rc != TWELL_OK) return rc;
  const Geometry g = geometry(shape);
  if ((rc = check_ell(out, g.n_rows)) != TWELL_OK) return rc;
  if ((g.n_rows > 0 && h == nullptr) || workspace == nullptr) return TWELL_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(workspace)) return TWELL_ERR_INVALID_ARG;
  if (workspace_bytes < pack_ws_bytes(shape)) return TWELL_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const PackWorkspace w = carve(shape, workspace, false);
  return hip_status(launch_ell_pack(g, elem_bytes(shape->dtype), h, w.route, out->values,
                                    out->columns, out->counts, out->dense_rows, out->dense_values,
                                    out->dense_capacity, out->n_dense, d_status, st));
}

TWELL_EXPORT int ell_unpack(const twell_shape* shape, const twell_ell* in, void* h, void* stream) {
  int rc = check_ell_shape(shape, false);
  if (rc != TWELL_OK) return rc;
  const Geometry g = geometry(shape);
  if ((rc = check_ell(in, g.n_rows)) != TWELL_OK) return rc;
  if (g.n_rows > 0 && h == nullptr) return TWELL_ERR_INVALID_ARG;
  if (!aligned16(h)) return TWELL_ERR_INVALID_ARG;
  if (ell_unpack_lds_bytes(g, elem_bytes(shape->dtype)) > 64 * 1024) return TWELL_ERR_UNSUPPORTED;
  return hip_status(launch_ell_unpack(g, elem_bytes(shape->dtype), in->values, in->columns,
                                      in->counts, in->dense_rows, in->dense_values, in->n_dense,
                                      in->dense_capacity, h, static_cast<hipStream_t>(stream)));
}

TWELL_EXPORT int ell_spmm(const twell_shape* shape, const twell_ell* in, const void* w_down,
                          void* y, void* stream) {
  int rc = check_ell_shape(shape, true);
  if (rc != TWELL_OK) return rc;
  const Geometry g = geometry(shape);
  if ((rc = check_ell(in, g.n_rows)) != TWELL_OK) return rc;
  if (g.n_rows > 0 && (w_down == nullptr || y == nullptr)) return TWELL_ERR_INVALID_ARG;
  if (!aligned16(w_down) || !aligned16(y)) return TWELL_ERR_INVALID_ARG;
  if (g.n_rows == 0) return TWELL_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int eb = elem_bytes(shape->dtype);
  // the ELL rows (a row listed among the stored dense rows is skipped) ...
  const DenseSkip skip{in->dense_rows, in->n_dense, in->dense_capacity};
  TWELL_TRY(launch_ell_spmm_sparse(g, eb, in->values, in->columns, in->counts, skip, w_down, y,
                                   st));
  // ... and the stored dense rows by the dense fallback GEMM
  if (eb == 2)
    TWELL_TRY(launch_fallback_bf16(g, static_cast<const uint16_t*>(in->dense_values),
                                   in->dense_rows, in->n_dense, in->dense_capacity,
                                   static_cast<const uint16_t*>(w_down), static_cast<uint16_t*>(y),
                                   st));
  else
    TWELL_TRY(launch_fallback_f32(g, static_cast<const float*>(in->dense_values), in->dense_rows,
                                  in->n_dense, in->dense_capacity,
                                  static_cast<const float*>(w_down), static_cast<float*>(y), st));
  return TWELL_OK;
}

// ------------------------------------------------------------------ backward
namespace twell {
namespace {

// The backward's shape rules on top of check_shape: every entry's place fits
// an int32.
int check_backward_shape(const twell_shape* s, int64_t dense_capacity) {
  int rc = check_shape(s, true);
  if (rc != TWELL_OK) return rc;
  if (dense_capacity < 0) return TWELL_ERR_INVALID_ARG;
  if (bwd_max_entries(geometry(s), dense_capacity) > INT32_MAX) return TWELL_ERR_UNSUPPORTED;
  if (!bwd_supported(geometry(s), elem_bytes(s->dtype))) return TWELL_ERR_UNSUPPORTED;
  return TWELL_OK;
}

}  // namespace
}  // namespace twell

TWELL_EXPORT size_t ffn_sparse_backward_workspace_size(const twell_shape* shape,
                                                       int64_t dense_capacity) {
  if (check_backward_shape(shape, dense_capacity) != TWELL_OK) return 0;
  return bwd_carve(geometry(shape), elem_bytes(shape->dtype), dense_capacity, nullptr).bytes;
}

TWELL_EXPORT int ffn_sparse_backward(const twell_shape* shape, const void* x, const void* w_up_t,
                                     const void* w_down, const twell_hybrid* h, const void* dy,
                                     void* dx, float* dw_up_t, float* db_up, float* dw_down,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape, true);
  if (rc != TWELL_OK) return rc;
  const Geometry g = geometry(shape);
  if ((rc = check_hybrid(h, g.n_rows)) != TWELL_OK) return rc;
  if ((rc = check_backward_shape(shape, h->dense_capacity)) != TWELL_OK) return rc;
  if (dw_up_t == nullptr || db_up == nullptr || dw_down == nullptr || workspace == nullptr)
    return TWELL_ERR_INVALID_ARG;
  if (g.n_rows > 0 &&
      (x == nullptr || w_up_t == nullptr || w_down == nullptr || dy == nullptr || dx == nullptr))
    return TWELL_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_up_t) || !aligned16(w_down) || !aligned16(dy) ||
      !aligned16(dx) || !aligned16(dw_up_t) || !aligned16(db_up) || !aligned16(dw_down) ||
      !aligned16(workspace))
    return TWELL_ERR_INVALID_ARG;
  const int eb = elem_bytes(shape->dtype);
  const BwdWorkspace w = bwd_carve(g, eb, h->dense_capacity, workspace);
  if (workspace_bytes < w.bytes) return TWELL_ERR_WORKSPACE;
  const BwdHybrid hy{h->values,       h->indices, h->counts,         h->dense_rows,
                     h->dense_values, h->n_dense, h->dense_capacity};
  return hip_status(launch_backward(g, eb, hy, x, w_up_t, w_down, dy, w, dx, dw_up_t, db_up,
                                    dw_down, static_cast<hipStream_t>(stream)));
}
