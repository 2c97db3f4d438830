// tsp_attn_fwd_bf16.hip -- the bf16 attention forward kernels (attn_fwd_bf16.h): their
// tile configuration per head dim and their launches. A translation unit of its own so
// that its code-generation flags (no NaN-quieting in the row maxima, MFMA results in arch
// VGPRs, the memory-clause scheduling strategy) apply to these kernels only; argument
// checks and the C ABI are in tsp_attn.hip.
#include <hip/hip_runtime.h>

#include "attn_fwd_bf16.h"
#include "host_common.h"

namespace {

using tsp_host::KernelShape;

// Tile configuration of the bf16 kernels per head dim and launch form (NR: 1 one key range,
// 2 two ranges, 3 the ring sweep): waves per workgroup, 32-row query blocks per wave, depth
// of the LDS stage ring, 32-key steps per stage, target waves per SIMD.
// dh 128: one-range launches run one wave per SIMD with two row blocks each (the fixed-max
// sweep in a pinned issue order, at half the LDS reads per product); two-range and ring
// launches, whose sweeps are short and whose masked diagonal steps weigh more, keep two
// waves per SIMD with one row block. Both have 8 row blocks per workgroup, so the host's
// tile plan (kernel shape) is the same for every form.
#ifndef TSP_DH128_NW
#define TSP_DH128_NW 4
#endif
#ifndef TSP_DH128_NBUF
#define TSP_DH128_NBUF 4
#endif
#ifndef TSP_DH128_SPS
#define TSP_DH128_SPS 1
#endif
#ifndef TSP_DH128_RB
#define TSP_DH128_RB 2
#endif
#ifndef TSP_DH128_OCC
#define TSP_DH128_OCC 1
#endif
struct CfgWave2 {  // dh 128, two waves per SIMD
  static constexpr int NW = 8, RB = 1, NBUF = 5, SPS = 2, OCC = 2;
};
template <int DH, int NR>
struct Bf16Cfg;
template <int NR>
struct Bf16Cfg<64, NR> {
  static constexpr int NW = 4, RB = 2, NBUF = 4, SPS = 1, OCC = 1;
};
template <>
struct Bf16Cfg<128, 1> {
  static constexpr int NW = TSP_DH128_NW, RB = TSP_DH128_RB, NBUF = TSP_DH128_NBUF, SPS = TSP_DH128_SPS,
                       OCC = TSP_DH128_OCC;
};
template <>
struct Bf16Cfg<128, 2> : CfgWave2 {};
template <>
struct Bf16Cfg<128, 3> : CfgWave2 {};
template <int NR>
struct Bf16Cfg<256, NR> {
  static constexpr int NW = 4, RB = 1, NBUF = 4, SPS = 1, OCC = 1;
};

template <int DH>
KernelShape shape_of() {
  using C = Bf16Cfg<DH, 1>;
  static_assert(C::NW * C::RB == Bf16Cfg<DH, 2>::NW * Bf16Cfg<DH, 2>::RB &&
                    C::NW * C::RB == Bf16Cfg<DH, 3>::NW * Bf16Cfg<DH, 3>::RB,
                "every launch form has the same row blocks per workgroup");
  static_assert(tsp::Bf16Stage<DH, C::NW, C::NBUF, C::SPS>::BK == 32, "32-key steps");
  return KernelShape{tsp::Bf16Stage<DH, C::NW, C::NBUF, C::SPS>::BK, C::NW, C::RB};
}

template <int DH, int NR, typename C = Bf16Cfg<DH, NR>>
void launch(const TspParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((tsp::attn_fwd_bf16_kernel<DH, C::NW, C::RB, C::NBUF, C::SPS, C::OCC, NR>), dim3(p.n_units),
                     dim3(C::NW * 64), 0, stream, p);
}

// dh 128, one key range: the one-wave form pays off over long sweeps; a range shorter
// than this (a gathered chunk, say) runs faster in the two-wave form, whose prologue,
// epilogue and masked steps cost less.
#ifndef TSP_DH128_ONE_WAVE_MIN_KEYS
#define TSP_DH128_ONE_WAVE_MIN_KEYS 8192
#endif
void launch_dh128_one_range(const TspParams& p, hipStream_t stream) {
  if ((int64_t)p.kv_hi - p.kv_lo >= TSP_DH128_ONE_WAVE_MIN_KEYS) launch<128, 1>(p, stream);
  else launch<128, 1, CfgWave2>(p, stream);
}

}  // namespace

namespace tsp_host {

bool bf16_kernel_shape(int64_t dh, KernelShape* ks) {
  switch (dh) {
    case 64: *ks = shape_of<64>(); return true;
    case 128: *ks = shape_of<128>(); return true;
    case 256: *ks = shape_of<256>(); return true;
  }
  return false;
}

bool launch_fwd_bf16(const TspParams& p, int64_t dh, hipStream_t stream) {
  const bool two = p.kv_hi2 > p.kv_lo2;  // two key ranges in one sweep
  switch (dh) {
    case 64: two ? launch<64, 2>(p, stream) : launch<64, 1>(p, stream); return true;
    case 128: two ? launch<128, 2>(p, stream) : launch_dh128_one_range(p, stream); return true;
    case 256: two ? launch<256, 2>(p, stream) : launch<256, 1>(p, stream); return true;
  }
  return false;
}

bool launch_fwd_bf16_ring(const TspParams& p, int64_t dh, hipStream_t stream) {
  switch (dh) {
    case 64: launch<64, 3>(p, stream); return true;
    case 128: launch<128, 3>(p, stream); return true;
    case 256: launch<256, 3>(p, stream); return true;
  }
  return false;
}

}  // namespace tsp_host
