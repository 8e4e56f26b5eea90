// Occupancy caps for the streaming kernels on gfx950 (host side).
//
// A CU holds as many blocks of a launch as its wave slots (8 per SIMD), its
// VGPRs and its 160 KiB of LDS allow, and LDS goes to blocks in 1280-byte
// units.  Measured on MI355X with one timestamp per wave: blocks asking for
// 6400 B of LDS run at most 25 to a CU, 7680 B 21, 10240 B 16, 23040 B 7,
// 32000 B 5 and 40960 B 4, with no other limit in the way.  Requesting LDS
// that a kernel never touches therefore caps the blocks per CU, which is the
// only use made of it here.
//
// With every wave slot filled, the packed kernels (3 KiB of loads per wave)
// and the plain streaming references (1 KiB) keep more reads in flight than
// HBM serves best once a launch fills the chip many times over; fewer waves
// per CU then move the same bytes faster.  The measurements are in the files
// that use these caps.  The fused prologue is not capped: every cap tried
// made it slower (its Q waves wait on a position -> cos/sin round trip as
// well as on their head).
#pragma once

namespace fp8kv {

constexpr int kLdsPerCu = 163840;   // bytes of LDS per CU
constexpr int kLdsUnit = 1280;      // allocation unit
constexpr int kMaxStaticLds = 1024; // a capped kernel's own LDS may not exceed this

constexpr int lds_allocated(int bytes) {
  return (bytes + kLdsUnit - 1) / kLdsUnit * kLdsUnit;
}

// Dynamic LDS (bytes) to request so that a CU holds at most `blocks_per_cu`
// blocks of a kernel whose static LDS is at most kMaxStaticLds; 0 = no cap.
// The request stops kMaxStaticLds short of a whole number of units, so the
// kernel's own LDS, whatever it is up to that bound, lands in the same units.
constexpr int lds_for_blocks_per_cu(int blocks_per_cu) {
  return blocks_per_cu <= 0
             ? 0
             : (kLdsPerCu / blocks_per_cu) / kLdsUnit * kLdsUnit - kMaxStaticLds;
}

constexpr bool cap_holds(int blocks_per_cu) {
  return kLdsPerCu / lds_allocated(lds_for_blocks_per_cu(blocks_per_cu)) == blocks_per_cu &&
         kLdsPerCu / lds_allocated(lds_for_blocks_per_cu(blocks_per_cu) + kMaxStaticLds) ==
             blocks_per_cu;
}
static_assert(cap_holds(25) && cap_holds(16) && cap_holds(7) && cap_holds(5) && cap_holds(4),
              "LDS request does not give the intended blocks per CU");

}  // namespace fp8kv
