// Layout constants of the CSR row plan (see plan.hip).
#pragma once

namespace sa {

constexpr int kPlanMagic = 0x53415031;  // "SAP1"
constexpr int kPlanHeaderWords = 8;     // magic, n, nnz lo, nnz hi, seg, items, 0, 0
constexpr int kPlanSeg = 512;           // maximum entries per segment

}  // namespace sa
