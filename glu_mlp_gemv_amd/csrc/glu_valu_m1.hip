// Instantiations of the VALU GEMV (glu_valu.h) for M = 1 hidden rows.
#include "glu_valu.h"

namespace glu {

ValuFn valu_pick_1(int R, int U, int NB, bool ragged, bool diag)
{
    if (diag) {
        if (R == 1) return valu_pick_m<1, 1, true>(U, NB, ragged);
        if (R == 2) return valu_pick_m<1, 2, true>(U, NB, ragged);
        return nullptr;
    }
    if (R == 1) return valu_pick_m<1, 1>(U, NB, ragged);
    if (R == 2) return valu_pick_m<1, 2>(U, NB, ragged);
    return nullptr;
}

}  // namespace glu
