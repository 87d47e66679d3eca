// The numeric constants of libmole, one copy each: the kernels read these
// arrays and the host helpers (mole_nf3_levels, mole_nf3_midpoints,
// mole_nf4_levels, mole_nf4_midpoints, mole_gelu_phi_coefficients) copy the
// same arrays out, so a test of the host copy pins what the device uses.
#pragma once

#include <stdint.h>

namespace mole {

// NF3 reconstruction levels (results section of the MoLE page: the table is
// compressed to 3 bits, e.g. NF3).  The NormalFloat construction at 3 bits:
// Phi^-1 at evenly spaced probabilities (4 positive levels, 3 negative, an
// exact zero), normalised to [-1, 1], rounded to fp32; code c -> level c.
constexpr uint32_t kNf3LevelBits[8] = {0xbf800000u, 0xbf08f740u, 0xbe7cdb98u, 0x00000000u,
                                       0x3e3bbcd2u, 0x3ec394b6u, 0x3f1f7bfeu, 0x3f800000u};
// Decision thresholds of the NF3 encoder: fp32 nearest-even rounding of the
// exact midpoint of two neighbouring fp32 levels.
constexpr uint32_t kNf3MidBits[7] = {0xbf447ba0u, 0xbec82e26u, 0xbdfcdb98u, 0x3dbbbcd2u,
                                     0x3e90b990u, 0x3f00a32cu, 0x3f4fbdffu};

// NF4: the same construction at 4 bits (8 positive levels, 7 negative, zero
// at code 7), and its thresholds built the same way.
constexpr uint32_t kNf4LevelBits[16] = {0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu,
                                        0xbe91a24bu, 0xbe3d353du, 0xbdba7869u, 0x00000000u,
                                        0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
                                        0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};
constexpr uint32_t kNf4MidBits[15] = {0xbf591cd8u, 0xbf1c5270u, 0xbeeb847du, 0xbeadea74u, 0xbe703ceau,
                                      0xbe0d38b9u, 0xbd3a7869u, 0x3d22fb01u, 0x3df64860u, 0x3e5067dcu,
                                      0x3e9582d2u, 0x3ec753f6u, 0x3f006d02u, 0x3f248dacu, 0x3f5c89d8u};

// Normal CDF for the bf16 GELU, u * Phi(u) (exact erf form of GELU).
// Phi(u) - 1/2 is odd; on [-kPhiPolyRange, kPhiPolyRange] it is the odd
// polynomial s * (c0 + c1 s^2 + ... + c9 s^18), s = u / kPhiPolyRange, whose
// coefficients are the fp32 rounding of the least-squares fit to Phi - 1/2
// on 4000 Chebyshev nodes of the interval (fp64 fit).  Evaluated in fp32 by
// Horner's rule its error is below 1e-5 there; outside, u is clamped to the
// interval first, an error of at most 1 - Phi(4) = 3.2e-5.  The build
// rounds GELU's output to bf16 (relative 2^-9) right after, so the
// approximation does not show.
constexpr float kPhiPolyRange = 4.0f;
constexpr int kPhiPolyTerms = 10;
constexpr float kPhiPolyCoef[kPhiPolyTerms] = {
    1.595752358e+00f, -4.254103661e+00f, 1.018382359e+01f, -1.914556694e+01f, 2.843501091e+01f,
    -3.288965607e+01f, 2.834799385e+01f, -1.688562202e+01f, 6.118065357e+00f, -1.005731821e+00f};

}  // namespace mole
