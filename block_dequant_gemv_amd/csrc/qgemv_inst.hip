// qgemv_inst.hip -- one translation unit of quantised GEMV instantiations.
// The build compiles this file once per (qtype, activation rows) pair, with
// QG_INST_QT set to the qtype (qgl::kQ8_0 ... kQ6_K) and QG_INST_M to 1 (the
// single-row calls: plain, gate|up, affine, RMSNorm prologue) or 2..6 (verify),
// so that the instantiations compile in parallel.
#include "qgemv_device.h"

#if !defined(QG_INST_QT) || !defined(QG_INST_M)
#error "build with -DQG_INST_QT=<qtype> -DQG_INST_M=<1..6>"
#endif

namespace qgk {

#if QG_INST_M == 1
template hipError_t launch_qgemv_m1<QG_INST_QT>(int, const QPlan &, const uint8_t *, const float *, float *,
                                                const QArgs &, hipStream_t);
#else
template hipError_t launch_qgemv_rows<QG_INST_QT, QG_INST_M>(const QPlan &, const uint8_t *, const float *, float *,
                                                             const QArgs &, hipStream_t);
#endif

}  // namespace qgk
