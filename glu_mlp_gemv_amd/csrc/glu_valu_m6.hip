// Instantiations of the VALU GEMV (glu_valu.h) for M = 6 hidden rows.
#include "glu_valu.h"

namespace glu {

ValuFn valu_pick_6(int R, int U, int NB, bool ragged)
{
    if (R == 1) return valu_pick_m<6, 1>(U, NB, ragged);
    return nullptr;
}

}  // namespace glu
